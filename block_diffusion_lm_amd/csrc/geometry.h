// geometry.h -- visible intervals and tile enumeration of the block-diffusion
// mask (and of the causal yardstick), shared by the kernels and by the host
// inspection entry points.
//
// Fast Diffusion Attention, "Block diffusion in one picture": a sample is
// [noisy | clean], each half of n tokens cut into consecutive blocks of b
// tokens (the last one shorter when b does not divide n).  A noisy query in
// block i sees the noisy keys of block i and the clean keys of blocks < i;
// a clean query in block i sees the clean keys of blocks <= i; a clean query
// sees no noisy key.  "Visit only the visible tiles": every half is tiled on
// its own, and a query tile only touches the key tiles that meet its rows'
// visible intervals (and, in the backward pass, a key tile only the query
// tiles whose rows see it); only tiles that some invisible pair crosses
// apply the mask element by element.
//
// Positions p are indices inside a half, 0 <= p < n.  The causal yardstick
// is a single half of length n ("clean") with block size 1, so that query p
// sees keys [0, p + 1).
//
// All visible intervals are of the form [lo(p), hi(p)) with lo and hi
// non-decreasing in the query row p, and the union over consecutive rows is
// contiguous; the rectangle classification below relies on both.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#define BD_HD __host__ __device__ __forceinline__
#else
#define BD_HD static inline
#endif

namespace bd {

enum : int { MODE_DIFFUSION = 0, MODE_CAUSAL = 1 };
enum : int { NOISY = 0, CLEAN = 1 };
enum : int { TILE_SKIP = 0, TILE_FULL = 1, TILE_PARTIAL = 2 };

struct Geom {
  int n;  // half length (diffusion) or sequence length (causal)
  int b;  // block size; 1 for causal

  BD_HD int bstart(int p) const { return (p / b) * b; }
  BD_HD int bend(int p) const {
    int s = (p / b) * b;
    return (b >= n - s) ? n : s + b;
  }
};

// Visible keys inside key half kh of a query row of half qh whose block is
// [bs, be): [lo, hi).
BD_HD void row_interval_of_block(int qh, int kh, int bs, int be, int& lo, int& hi) {
  lo = (qh == NOISY && kh == NOISY) ? bs : 0;  // own noisy block, both directions
  hi = (qh == NOISY) ? (kh == NOISY ? be       // ... up to the end of the block
                                    : bs)      // clean blocks strictly before own block
                     : (kh == CLEAN ? be       // clean blocks up to and including own block
                                    : 0);      // clean rows see no noisy key
}

// Visible keys of query row p (half qh) inside key half kh: [lo, hi); the
// same as row_interval_of_block with p's block (tests/test_geometry_header.py
// checks this exhaustively on small shapes).
BD_HD void row_interval(const Geom& g, int qh, int kh, int p, int& lo, int& hi) {
  if (qh == NOISY && kh == NOISY) {        // own noisy block, both directions
    lo = g.bstart(p);
    hi = g.bend(p);
  } else if (qh == NOISY) {                 // clean blocks strictly before own block
    lo = 0;
    hi = g.bstart(p);
  } else if (kh == CLEAN) {                 // clean blocks up to and including own block
    lo = 0;
    hi = g.bend(p);
  } else {                                  // clean rows see no noisy key
    lo = 0;
    hi = 0;
  }
}

// Query rows of half qh that see a key of half kh whose block is
// [bs, be): [lo, hi).
BD_HD void col_interval_of_block(int n, int qh, int kh, int bs, int be, int& lo, int& hi) {
  if (kh == NOISY && qh == NOISY) {
    lo = bs;
    hi = be;
  } else if (kh == CLEAN && qh == NOISY) {  // noisy rows of later blocks
    lo = be;
    hi = n;
  } else if (kh == CLEAN) {                 // clean rows of the same or later blocks
    lo = bs;
    hi = n;
  } else {
    lo = 0;
    hi = 0;
  }
}

// Query rows of half qh that see key c of half kh: [lo, hi).
BD_HD void col_interval(const Geom& g, int qh, int kh, int c, int& lo, int& hi) {
  col_interval_of_block(g.n, qh, kh, g.bstart(c), g.bend(c), lo, hi);
}

// Classify the rectangle rows [r0, r1) x keys [c0, c1) (r0 < r1 <= n,
// c0 < c1; c1 may pass n for a ragged last tile, and keys >= n count as
// invisible).  Monotone intervals make the rows r0 and r1 - 1 decisive.
BD_HD int classify(const Geom& g, int qh, int kh, int r0, int r1, int c0, int c1) {
  int lo_first, hi_first, lo_last, hi_last;
  row_interval(g, qh, kh, r0, lo_first, hi_first);
  row_interval(g, qh, kh, r1 - 1, lo_last, hi_last);
  if (c0 >= hi_last || c1 <= lo_first) return TILE_SKIP;
  if (lo_last <= c0 && c1 <= hi_first) return TILE_FULL;
  return TILE_PARTIAL;
}

BD_HD int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Forward enumeration: the key tiles (of tn keys) visited by query tile qt
// (of tm rows) of half qh.  At most two segments, each a contiguous range of
// key tiles in one key half.  For noisy rows the noisy segment (the block
// diagonal) comes first, then the clean context.  (Plain fields rather than
// arrays: a runtime-indexed array here would be placed in memory by the
// device compiler.)
struct Segments {
  int count;
  int half0, begin0, end0;
  int half1, begin1, end1;
  BD_HD int half(int i) const { return i ? half1 : half0; }
  BD_HD int begin(int i) const { return i ? begin1 : begin0; }
  BD_HD int end(int i) const { return i ? end1 : end0; }
  BD_HD int tiles() const { return (count > 0 ? end0 - begin0 : 0) + (count > 1 ? end1 - begin1 : 0); }
};

// Append the range [begin, end) of half h if it is not empty.
BD_HD void push_segment(Segments& s, int h, int begin, int end) {
  if (end <= begin) return;
  if (s.count == 0) {
    s.half0 = h;
    s.begin0 = begin;
    s.end0 = end;
  } else {
    s.half1 = h;
    s.begin1 = begin;
    s.end1 = end;
  }
  ++s.count;
}

BD_HD Segments empty_segments() {
  Segments s = {0, CLEAN, 0, 0, CLEAN, 0, 0};
  return s;
}

BD_HD Segments fwd_segments(const Geom& g, int mode, int qh, int qt, int tm, int tn) {
  Segments s = empty_segments();
  const int r0 = qt * tm;
  const int r1 = (tm >= g.n - r0) ? g.n : r0 + tm;
  int lo_first, hi_first, lo_last, hi_last;
  if (mode == MODE_DIFFUSION && qh == NOISY) {
    row_interval(g, qh, NOISY, r0, lo_first, hi_first);
    row_interval(g, qh, NOISY, r1 - 1, lo_last, hi_last);
    if (hi_last > lo_first) push_segment(s, NOISY, lo_first / tn, ceil_div(hi_last, tn));
  }
  row_interval(g, qh, CLEAN, r0, lo_first, hi_first);
  row_interval(g, qh, CLEAN, r1 - 1, lo_last, hi_last);
  if (hi_last > lo_first) push_segment(s, CLEAN, lo_first / tn, ceil_div(hi_last, tn));
  return s;
}

// Backward enumeration: the query tiles (of tm rows) that see key tile kt
// (of tn keys) of half kh.  Clean keys are seen by clean rows first, then by
// noisy rows of later blocks; noisy keys only by noisy rows of their block.
BD_HD Segments bwd_segments(const Geom& g, int mode, int kh, int kt, int tm, int tn) {
  Segments s = empty_segments();
  const int c0 = kt * tn;
  const int c1 = (tn >= g.n - c0) ? g.n : c0 + tn;
  int lo_first, hi_first, lo_last, hi_last;
  if (mode == MODE_CAUSAL || kh == CLEAN) {
    col_interval(g, CLEAN, kh, c0, lo_first, hi_first);
    col_interval(g, CLEAN, kh, c1 - 1, lo_last, hi_last);
    if (hi_last > lo_first) push_segment(s, CLEAN, lo_first / tm, ceil_div(hi_last, tm));
  }
  if (mode == MODE_DIFFUSION) {
    col_interval(g, NOISY, kh, c0, lo_first, hi_first);
    col_interval(g, NOISY, kh, c1 - 1, lo_last, hi_last);
    if (hi_last > lo_first) push_segment(s, NOISY, lo_first / tm, ceil_div(hi_last, tm));
  }
  return s;
}

}  // namespace bd
