// Tile classification shared by the kernels and the host planner.
//
// The visibility rule of one (query i, key j) pair is the AND of the enabled
// predicates (triton_kernels.py page, forward kernel: segment equality,
// i >= j, j > i - W; mosaic_backward.py page, ranker_mask_mosaic_kv_q:
// (j in hist and (i in hist or i in cand)) or (i in cand and j == i)).
// Which tiles to visit is derived here from those element predicates, so a
// tile is skipped only if it holds no visible pair, and every tile is visited
// at most once, whatever the tile sizes, window length or ranker split.
#pragma once

#if defined(__HIPCC__)
#define ATTN_HD __host__ __device__ inline
#else
#define ATTN_HD inline
#endif

namespace attn {

enum TileClass { TILE_EMPTY = 0, TILE_FULL = 1, TILE_PARTIAL = 2 };

struct MaskSpec {
  int L;
  int causal;
  int window;           // 0: off
  int ranker;           // 0: off
  int hl, hu, cl, cu;   // ranker bounds of this batch row
  int has_seg;          // segment ids present (tiles with them are never FULL)
};

ATTN_HD int imin(int a, int b) { return a < b ? a : b; }
ATTN_HD int imax(int a, int b) { return a > b ? a : b; }

// Interval [a0, a1) intersects [b0, b1)?
ATTN_HD bool overlaps(int a0, int a1, int b0, int b1) { return imax(a0, b0) < imin(a1, b1); }
// [a0, a1) contained in [b0, b1)?
ATTN_HD bool inside(int a0, int a1, int b0, int b1) { return a0 >= b0 && a1 <= b1; }

// Element predicate without segments.
ATTN_HD bool pair_visible(int i, int j, const MaskSpec& s) {
  bool ok = (i < s.L) && (j < s.L) && (i >= 0) && (j >= 0);
  if (s.causal) ok = ok && (j <= i);
  if (s.window > 0) ok = ok && (j > i - s.window);
  if (s.ranker) {
    bool qh = i >= s.hl && i < s.hu, qc = i >= s.cl && i < s.cu;
    bool kh = j >= s.hl && j < s.hu, kc = j >= s.cl && j < s.cu;
    ok = ok && ((kh && (qh || qc)) || (qc && kc && i == j));
  }
  return ok;
}

// Class of the block rows [q0, q1) x keys [k0, k1) under causal / window /
// ranker / length, ignoring segment ids (the caller handles those).  EMPTY is
// exact for each predicate alone and therefore sound for their AND; FULL is
// only returned when every pair is visible.
ATTN_HD int tile_class(int q0, int q1, int k0, int k1, const MaskSpec& s) {
  // FULL means every element of the unclipped block is a visible pair, so a
  // block reaching past L is at best PARTIAL.
  bool full = q1 <= s.L && k1 <= s.L;
  q1 = imin(q1, s.L);
  k1 = imin(k1, s.L);
  if (q0 >= q1 || k0 >= k1) return TILE_EMPTY;
  if (s.causal) {
    if (k0 > q1 - 1) return TILE_EMPTY;          // every key after every row
    full = full && (k1 - 1 <= q0);
  }
  if (s.window > 0) {
    if (k1 - 1 < q0 - s.window + 1) return TILE_EMPTY;   // every key too old
    full = full && (k0 >= (q1 - 1) - s.window + 1);
  }
  if (s.ranker) {
    bool rows_active = overlaps(q0, q1, s.hl, s.hu) || overlaps(q0, q1, s.cl, s.cu);
    bool hist_pairs = rows_active && overlaps(k0, k1, s.hl, s.hu);
    // diagonal pairs: i == j in rows, keys and candidates
    int d0 = imax(imax(q0, k0), s.cl), d1 = imin(imin(q1, k1), s.cu);
    bool diag_pairs = d0 < d1;
    if (!hist_pairs && !diag_pairs) return TILE_EMPTY;
    bool rows_all_active;
    if (inside(q0, q1, s.hl, s.hu) || inside(q0, q1, s.cl, s.cu)) {
      rows_all_active = true;
    } else if (s.hl <= s.cl && s.cl <= s.hu) {
      rows_all_active = inside(q0, q1, s.hl, imax(s.hu, s.cu));
    } else if (s.cl <= s.hl && s.hl <= s.cu) {
      rows_all_active = inside(q0, q1, s.cl, imax(s.hu, s.cu));
    } else {
      rows_all_active = false;
    }
    full = full && rows_all_active && inside(k0, k1, s.hl, s.hu);
  }
  if (s.has_seg) full = false;
  return full ? TILE_FULL : TILE_PARTIAL;
}

// Contiguous range of key tiles (tile size bn) that can hold a visible pair
// for rows [q0, q1): causal and window bounds only.  Returns false if empty.
ATTN_HD bool key_tile_range(int q0, int q1, int bn, const MaskSpec& s, int* t0, int* t1) {
  q1 = imin(q1, s.L);
  if (q0 >= q1) return false;
  int kmin = 0, kmax = s.L - 1;
  if (s.window > 0) kmin = imax(kmin, q0 - s.window + 1);
  if (s.causal) kmax = imin(kmax, q1 - 1);
  if (kmin > kmax) return false;
  *t0 = kmin / bn;
  *t1 = kmax / bn + 1;
  return true;
}

// Contiguous range of query tiles (tile size bm) that can see keys [k0, k1).
ATTN_HD bool query_tile_range(int k0, int k1, int bm, const MaskSpec& s, int* t0, int* t1) {
  k1 = imin(k1, s.L);
  if (k0 >= k1) return false;
  int qmin = 0, qmax = s.L - 1;
  if (s.causal) qmin = imax(qmin, k0);
  if (s.window > 0) qmax = imin(qmax, (k1 - 1) + s.window - 1);
  if (qmin > qmax) return false;
  *t0 = qmin / bm;
  *t1 = qmax / bm + 1;
  return true;
}

}  // namespace attn

namespace attn {

// Stored dS tiles.  The stored-dS backward keeps dS (bf16) of every visited
// block of DS_T queries x DS_T keys, so the dQ contraction can read it
// instead of recomputing it.  A tile is four 8 KB groups of 32 keys (the
// keys of one dK/dV wave); a group is four 2 KB blocks of 32 queries, each
// two 1 KB halves in the order the dK/dV wave holds them: 16-byte chunk
// (key k, queries 8c .. 8c+7) of the group at byte ds_chunk_offset(k, c)
// (c = 0 .. 15).  Each store instruction of that wave then writes 1 KB of
// whole cache lines, and the dQ kernel loads a group with contiguous 1 KB
// loads; the key bits XORed into a chunk's slot make the dQ kernel's
// transposed LDS reads of it conflict-free on 64 banks (per 32 lanes).
// Query tile qt of one (batch row, query head) owns the slots of its key-tile
// band [ds_lo(qt), ds_hi(qt)), the key_tile_range of causal and window bounds
// (identical for every batch row and head: ranker and segment skips only
// leave slots unused), packed one query tile after another.
constexpr int DS_T = 128;
constexpr int DS_ELEMS = DS_T * DS_T;
// Byte offset of chunk (key k, query chunk c) inside its 32-key group: block
// c / 4 (2 KB each), half (c / 2) % 2 of it (1 KB: one store instruction),
// then 16 bytes per slot 32 (c % 2) + (k ^ 4 (c % 2) ^ 8 ((c / 2) % 2)).
ATTN_HD int ds_chunk_offset(int k, int c) {
  const int pp = c & 1, hq = (c >> 1) & 1;
  return (c >> 2) * 2048 + hq * 1024 + (pp * 32 + (k ^ (pp << 2) ^ (hq << 3))) * 16;
}

struct DsBand {
  int nt;       // tiles per side, ceil(L / DS_T)
  int causal;
  int c;        // window: band reaches c tiles below the diagonal (nt when off)
};

ATTN_HD DsBand ds_band(int L, int causal, int window) {
  DsBand d;
  d.nt = (L + DS_T - 1) / DS_T;
  d.causal = causal;
  // first key of row q0 = DS_T qt is q0 - W + 1, in tile qt - ceil((W - 1) / DS_T)
  d.c = window > 0 ? (window + DS_T - 2) / DS_T : d.nt;
  return d;
}
ATTN_HD int ds_lo(int qt, const DsBand& d) { return imax(0, qt - d.c); }
ATTN_HD int ds_hi(int qt, const DsBand& d) { return d.causal ? qt + 1 : d.nt; }
// First slot of query tile qt: sum over earlier query tiles of the band widths.
ATTN_HD long long ds_offset(int qt, const DsBand& d) {
  const long long q = qt;
  const long long his = d.causal ? q * (q + 1) / 2 : q * d.nt;
  const long long n = q - 1 - d.c > 0 ? q - 1 - d.c : 0;   // rows with ds_lo > 0
  return his - n * (n + 1) / 2;
}
ATTN_HD long long ds_slots_per_head(const DsBand& d) { return ds_offset(d.nt, d); }
// Slot of block (qt, kt), or -1 outside the band.
ATTN_HD long long ds_slot(int qt, int kt, const DsBand& d) {
  if (kt < ds_lo(qt, d) || kt >= ds_hi(qt, d)) return -1;
  return ds_offset(qt, d) + (kt - ds_lo(qt, d));
}

}  // namespace attn
