// Drawing one token from a logit row by inverse CDF, with the chunk chosen
// from the stream pass's partials and only that chunk re-read (used by the
// linear and the tree finalize kernels).
#pragma once

#include "verify_common.h"

namespace specsam {
namespace {

// ---------------------------------------------------------------------------
// Draw from one row by inverse CDF in ascending token order: the first token
// whose running weight exceeds u * total (strict, so zero weights are never
// chosen). Weights are exp2((l - m) * kk) with token `excl` removed (one-hot
// residual; excl < 0 for the bonus), or, for RESIDUAL, max(0, exp2((l - m) *
// kk) / S - q).
//
// pick_chunk (one wavefront): the chunk weights, from the stream pass's
// partials, are scanned in chunk order and the first chunk whose running sum
// exceeds u * total is taken, with the target left inside it; if rounding
// leaves none, the last chunk with positive weight (its last positive token
// is then drawn). On the vector path the chunk weights are the sums of the
// stream pass's quarter sums, and pick_slice then takes the quarter (a
// contiguous quarter of the chunk's tokens) the same way. draw_in_chunk
// (whole workgroup): that chunk, or quarter, is re-read with the stream
// pass's layout, in which token order is (load, lane, element). Each lane
// sums its vectors; the (load, wavefront) cell totals (32 for a chunk, 8 for
// a quarter) are scanned in token order to find the cell, a wavefront scan
// inside the cell finds the lane, and that lane scans its vector. The cell
// totals and the lane scan come from the same inclusive scan arithmetic, so
// the search is consistent; a target beyond the re-read total (a rounding
// difference with the partials) takes the last positive weight re-read.
//
// Every weight is a float32 term, but the running sum over chunks, the
// target u * total and a chunk's rescale to the row max are taken in double:
// a float32 running sum over 2^17 tokens moves a breakpoint by a few float32
// roundings of the total, which at that many tokens is the width of many
// tokens' intervals. Inside the chosen chunk (one chunk's share of the
// total) the scans are float32: their rounding is that share of a float32
// ulp.
// ---------------------------------------------------------------------------
struct ChunkPick {
  int chunk;    // -1: every weight is 0
  double t_in;  // target left inside the chunk (the slice, when one is
                // chosen); +inf: take its last positive
  int slice;    // -1: the whole chunk; else the quarter that holds the
                // target (pick_slice)
};

// Weight of a chunk relative to the row max m: its partial sum s (relative
// to the chunk's own max mc) times exp2((mc - m) * kk). The exponent is
// formed in double (a float product would round it by up to 1e-6 for
// |exponent| ~ 20, an error shared by every token of the chunk); its integer
// part is applied exactly by ldexp and its fraction by the hardware exp2,
// whose error (about one float32 ulp) is that of any single term. A chunk
// whose max is -inf weighs 0; NaN (a non-finite row) stays NaN.
__device__ __forceinline__ double chunk_weight(float s, float mc, float m, float kk) {
  const double e = ((double)mc - (double)m) * (double)kk;
  if (e != e) return (double)NAN;
  if (e < -4096.0) return 0.0;  // below every double, -inf included
  const double fl = floor(e);
  const float fr = (float)(e - fl);  // in [0, 1)
  return ldexp((double)s * (double)fast_exp2(fr), (int)fl);
}

// A chunk split in quarters, in token order (quarter q: the stream layout's
// loads 2q and 2q + 1, 2 * 256 contiguous vectors), with weights w0..w3
// (double). The chunk's weight is (w0 + w1) + (w2 + w3), and the running
// sums in pick_slice are formed so that the last one is that same value: a
// target the chunk pick left below the chunk's weight always falls in a
// quarter.
// Scale of a chunk's sums (relative to its max mc) to the row max m:
// exp2((mc - m) * kk), as chunk_weight forms it (0 below every double, NaN
// for a NaN exponent).
__device__ __forceinline__ double chunk_scale(float mc, float m, float kk) {
  const double e = ((double)mc - (double)m) * (double)kk;
  if (e != e) return (double)NAN;
  if (e < -4096.0) return 0.0;
  const double fl = floor(e);
  return ldexp((double)fast_exp2((float)(e - fl)), (int)fl);
}
struct QuarterW {
  double w0, w1, w2, w3;
  __device__ double chunk() const { return (w0 + w1) + (w2 + w3); }
};
__device__ __forceinline__ void pick_slice(ChunkPick& pk, const QuarterW& q) {
  const double w0 = q.w0, w1 = q.w1, w2 = q.w2, w3 = q.w3;
  const double c1 = w0 + w1, c2 = c1 + w2, c3 = c1 + (w2 + w3);
  const double t = pk.t_in;
  // (scalar selects: an indexed local array would live in scratch memory)
  const int hit = w0 > t ? 0 : c1 > t ? 1 : c2 > t ? 2 : c3 > t ? 3 : -1;
  const int lastpos = w3 > 0.0 ? 3 : w2 > 0.0 ? 2 : w1 > 0.0 ? 1 : w0 > 0.0 ? 0 : -1;
  if (hit >= 0) {
    const double before = hit == 0 ? 0.0 : hit == 1 ? w0 : hit == 2 ? c1 : c2;
    pk.slice = hit;
    pk.t_in = fmax(0.0, t - before);
  } else {
    // Rounding put the target past the chunk: its last positive quarter,
    // and that quarter's last positive token.
    pk.slice = lastpos < 0 ? 3 : lastpos;
    pk.t_in = INFINITY;
  }
}

// One wavefront, all lanes active; weight(c) (a double) is called for c < nc.
template <typename WeightFn>
__device__ __forceinline__ ChunkPick pick_chunk(int nc, float u, WeightFn weight) {
  constexpr int kGroups = kMaxChunks / kWave;
  const int l = lane_id();
  double W[kGroups], cum[kGroups];
  double carry = 0.0;
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    W[g] = 0.0;
    cum[g] = carry;
    if (g * kWave < nc) {
      const int c = g * kWave + l;
      W[g] = c < nc ? (double)weight(c) : 0.0;
      cum[g] = wave_inclusive_sum_d(W[g]) + carry;
      carry = readlane_d(cum[g], 63);
    }
  }
  const double t = (double)u * carry;
  ChunkPick r{-1, INFINITY, -1};
  int lastpos = -1;
#pragma unroll
  for (int g = 0; g < kGroups; ++g) {
    if (g * kWave < nc) {
      const int c = g * kWave + l;
      const unsigned long long hit = __ballot(c < nc && cum[g] > t);
      const unsigned long long pos = __ballot(c < nc && W[g] > 0.0);
      if (hit && r.chunk < 0) {
        const int ln = __ffsll((unsigned long long)hit) - 1;
        r.chunk = g * kWave + ln;
        // The sum before this chunk (its running sum less its own weight)
        // can round above the previous chunk's running sum, which the
        // target did not exceed: the target then lies at the start of this
        // chunk, not before it.
        r.t_in = fmax(0.0, t - (readlane_d(cum[g], ln) - readlane_d(W[g], ln)));
      }
      if (pos) lastpos = g * kWave + 63 - __clzll((unsigned long long)pos);
    }
  }
  if (r.chunk < 0) r.chunk = lastpos;
  return r;
}

// pick_chunk over chunks given by their quarters, then pick_slice in the
// chosen chunk. Each lane forms the quarters of its own chunk among the first
// 64 once (a lane past nc forms the last chunk's, which the pick ignores);
// the chosen chunk's quarters then come from its lane instead of being
// formed (or fetched) again. The arithmetic is that of quarters(c) either
// way, so the pick is the same.
template <typename QuartersFn>
__device__ __forceinline__ ChunkPick pick_chunk_slice(int nc, float u, QuartersFn quarters) {
  const QuarterW mine = quarters(min(lane_id(), nc - 1));
  ChunkPick pk = pick_chunk(
      nc, u, [&](int c) { return c < kWave ? mine.chunk() : quarters(c).chunk(); });
  if (pk.chunk >= kWave) {
    pick_slice(pk, quarters(pk.chunk));
  } else if (pk.chunk >= 0) {
    const int ln = pk.chunk;
    pick_slice(pk, QuarterW{readlane_d(mine.w0, ln), readlane_d(mine.w1, ln),
                            readlane_d(mine.w2, ln), readlane_d(mine.w3, ln)});
  }
  return pk;
}

// draw_in_chunk's mark for a target past the chunk's re-read total.
constexpr int kDrawPastEnd = INT_MIN;

struct DrawShared {
  float cell[kLoads * kWaves];  // (load, wave) totals in token order
  int wlast[kWaves];            // each wavefront's last positive weight
  int result;
  float result_l;  // the drawn token's logit (NaN if the draw did not see it)
};

// Weight of a token with logit l (token index i); tokens below the
// truncation threshold lam have probability 0.
template <int DT, bool RESIDUAL, typename Excl>
__device__ __forceinline__ float draw_weight(float l, int i, Excl excl, float m,
                                             float kk, float invS, float qi,
                                             float lam) {
  const float w = (l >= lam) ? fast_exp2((l - m) * kk) : 0.0f;
  if constexpr (RESIDUAL)
    return fmaxf(0.0f, w * invS - qi);
  else
    return excl(i) ? 0.0f : w;
}

// q of a chunk for the residual, in the stream layout (element (it, k) of
// the lane is token elem_index(cstart, tid, it, k)); 0 past the row's end.
// NL = 2: the q of one quarter (draw_vec<true>).
template <int DT, int NL = kLoads>
struct QChunk {
  float v[NL][kVec<DT>];
  __device__ __forceinline__ float at(int it, int k) const { return v[it][k]; }
};
// No q (the draws from p).
struct NoQ {
  __device__ __forceinline__ float at(int, int) const { return 0.0f; }
};

// Requests every q value of the chunk at once: one load per vector, none
// behind a branch (an index past the row's end is clamped into the row).
// q_tail_zero then sets the values past the end to 0, once the kernel's
// loads are all requested (see load_chunk_flat).
template <int DT, bool VP>
__device__ __forceinline__ void load_q_chunk(const float* qrow, int cstart, int V, int tid,
                                             QChunk<DT>& q) {
  constexpr int kH = kVec<DT> / 4;  // 16-byte q vectors per logit vector
  if constexpr (VP) {
    // (V is a multiple of the logit vector width, so a vector is either
    // wholly in the row or wholly past its end)
    const int last = (V - cstart) / 4 - 1;  // the row's last q vector here
    const f32x4* p = reinterpret_cast<const f32x4*>(qrow + cstart);
#pragma unroll
    for (int it = 0; it < kLoads; ++it)
#pragma unroll
      for (int h = 0; h < kH; ++h) {
        const f32x4 x =
            __builtin_nontemporal_load(p + min((it * kThreads + tid) * kH + h, last));
#pragma unroll
        for (int k = 0; k < 4; ++k) q.v[it][4 * h + k] = x[k];
      }
  } else {
#pragma unroll
    for (int it = 0; it < kLoads; ++it)
#pragma unroll
      for (int k = 0; k < kVec<DT>; ++k)
        q.v[it][k] = qrow[min(elem_index<DT, false>(cstart, tid, it, k), V - 1)];
  }
}
template <int DT, bool VP>
__device__ __forceinline__ void q_tail_zero(int cstart, int V, int tid, QChunk<DT>& q) {
#pragma unroll
  for (int it = 0; it < kLoads; ++it)
#pragma unroll
    for (int k = 0; k < kVec<DT>; ++k)
      q.v[it][k] = elem_index<DT, VP>(cstart, tid, it, k) < V ? q.v[it][k] : 0.0f;
}

constexpr float kLn2 = 0.69314718055994531f;

// Log-probability of token `tok` drawn from row r: (l - m) / T - log S with
// the row's (m, S) at scale kk = log2(e) / T. lt is the token's logit as the
// draw saw it; NaN (a rounding fallback) reads it from the row.
template <int DT>
__device__ __forceinline__ float drawn_logprob(const Args& a, int b, int r, int tok,
                                               float lt, float m, float S, float kk) {
  if (tok < 0) return NAN;
  if (lt != lt)
    lt = load_one<DT>(a.logits + ((int64_t)b * (a.K + 1) + r) * a.V * Dt<DT>::kBytes,
                      tok);
  return ((lt - m) * kk - log2f(S)) * kLn2;
}

// Tokens a draw leaves out: one token (or none, -1) ...
struct OneToken {
  int t;
  __device__ __forceinline__ bool operator()(int i) const { return i == t; }
};

struct NoDuring {
  __device__ void operator()() const {}
};

// Requests the chosen chunk of row r (nothing if every weight is 0). On the
// vector path the loads are branch-free (clamped into the row, see
// load_chunk_flat) and draw_in_chunk sets the values past the row's end:
// load_chunk's two paths, joined here, made the compiler wait for every
// load in flight before the full-chunk path's loads.
// With a quarter chosen (vector path only) each thread requests two
// vectors: the stream layout's loads 2q and 2q + 1.
constexpr int kSliceLoads = 2;

// Vector index, within the chunk, of load `it` of this thread: the stream
// layout, for the whole chunk or from quarter qs on.
template <bool SLICE>
__device__ __forceinline__ int draw_vec(int it, int qs) {
  return ((SLICE ? 2 * qs : 0) + it) * kThreads + (int)threadIdx.x;
}

// The whole chunk (pk.slice < 0).
template <int DT, bool VP>
__device__ __forceinline__ void draw_load(const Args& a, int b, int r, ChunkPick pk,
                                          u32x4 (&raw)[kLoads]) {
  if (pk.chunk < 0) return;
  const unsigned char* row =
      a.logits + ((int64_t)b * (a.K + 1) + r) * a.V * Dt<DT>::kBytes;
  const int cstart = pk.chunk * kChunk<DT>;
  if constexpr (VP)
    load_chunk_flat<DT, false>(row, cstart, a.V, threadIdx.x, raw);
  else
    load_chunk<DT, VP, false>(row, cstart, a.V, threadIdx.x, raw);
}
// The chosen quarter (pk.slice >= 0, vector path). A separate array from
// the whole chunk's: one array written by both, with different lengths, was
// given a memory home by the compiler.
template <int DT>
__device__ __forceinline__ void draw_load_slice(const Args& a, int b, int r, ChunkPick pk,
                                                u32x4 (&rs)[kSliceLoads]) {
  if (pk.chunk < 0) return;
  const unsigned char* row =
      a.logits + ((int64_t)b * (a.K + 1) + r) * a.V * Dt<DT>::kBytes;
  const int cstart = pk.chunk * kChunk<DT>;
  const u32x4* p = reinterpret_cast<const u32x4*>(row + (int64_t)cstart * Dt<DT>::kBytes);
  const int last = (a.V - cstart) / kVec<DT> - 1;
#pragma unroll
  for (int it = 0; it < kSliceLoads; ++it) rs[it] = p[min(draw_vec<true>(it, pk.slice), last)];
}

// Whole workgroup; `pk` must be the same in every thread and `raw_in` hold the
// chunk draw_load requested. `during` runs first, while that chunk is still
// in flight (the fused step appends the accepted drafts to the automaton
// there).
// RESIDUAL: q holds the chunk's q (load_q_chunk), requested with `raw_in`.
// q of the chosen quarter qs (vector path), requested like load_q_chunk's,
// and its values past the row's end set to 0 once every load is requested.
template <int DT>
__device__ __forceinline__ void load_q_slice(const float* qrow, int cstart, int V, int qs,
                                             QChunk<DT, kSliceLoads>& q) {
  constexpr int kH = kVec<DT> / 4;
  const int last = (V - cstart) / 4 - 1;
  const f32x4* p = reinterpret_cast<const f32x4*>(qrow + cstart);
#pragma unroll
  for (int it = 0; it < kSliceLoads; ++it)
#pragma unroll
    for (int h = 0; h < kH; ++h) {
      const f32x4 x = __builtin_nontemporal_load(p + min(draw_vec<true>(it, qs) * kH + h, last));
#pragma unroll
      for (int k = 0; k < 4; ++k) q.v[it][4 * h + k] = x[k];
    }
}
template <int DT>
__device__ __forceinline__ void q_slice_tail_zero(int cstart, int V, int qs,
                                                  QChunk<DT, kSliceLoads>& q) {
#pragma unroll
  for (int it = 0; it < kSliceLoads; ++it)
#pragma unroll
    for (int k = 0; k < kVec<DT>; ++k)
      q.v[it][k] = cstart + draw_vec<true>(it, qs) * kVec<DT> + k < V ? q.v[it][k] : 0.0f;
}

// SLICE: pk.slice >= 0 and `raw_in` holds that quarter (draw_load_slice);
// the cells are then its 2 loads times 4 wavefronts, in token order as for
// a whole chunk.
template <int DT, bool VP, bool RESIDUAL, typename Excl, typename During = NoDuring,
          typename Q = NoQ, bool SLICE = false>
__device__ __forceinline__ int draw_in_chunk(const Args& a, DrawShared& sh, int b, int r,
                                             ChunkPick pk, Excl excl, float m, float kk,
                                             float invS, float lam,
                                             const u32x4 (&raw_in)[SLICE ? kSliceLoads : kLoads],
                                             During during = During{}, const Q& q = Q{}) {
  static_assert(!SLICE || VP, "quarters: vector path");
  constexpr int NL = SLICE ? kSliceLoads : kLoads;
  constexpr unsigned kNegInfWord = DT == SS_DTYPE_F32 ? 0xff800000u : 0xff80ff80u;
  const int tid = threadIdx.x, w = tid / kWave, l = tid % kWave;
  during();
  if (pk.chunk < 0) return -1;
  const int cstart = pk.chunk * kChunk<DT>;
  const int qs = SLICE ? pk.slice : 0;
  u32x4 raw[NL];
#pragma unroll
  for (int it = 0; it < NL; ++it) raw[it] = raw_in[it];
  if constexpr (VP) {
    // vectors past the row's end (their loads were clamped into the row)
    const int rem = a.V - cstart;
    if (rem < kChunk<DT>) {
#pragma unroll
      for (int it = 0; it < NL; ++it) {
        const bool in = draw_vec<SLICE>(it, qs) * kVec<DT> < rem;
        const u32x4 x = raw[it];
        raw[it] = u32x4{in ? x[0] : kNegInfWord, in ? x[1] : kNegInfWord,
                        in ? x[2] : kNegInfWord, in ? x[3] : kNegInfWord};
      }
    }
  }
  auto index = [&](int it, int k) {
    if constexpr (SLICE)
      return cstart + draw_vec<true>(it, qs) * kVec<DT> + k;
    else
      return elem_index<DT, VP>(cstart, tid, it, k);
  };
  const float t_in = (float)pk.t_in;
  auto weight = [&](int it, int k) {
    return draw_weight<DT, RESIDUAL>(elem<DT>(raw[it], k), index(it, k), excl, m, kk,
                                     invS, q.at(it, k), lam);
  };
  float vs[NL];
#pragma unroll
  for (int it = 0; it < NL; ++it) {
    float acc = 0.0f;
#pragma unroll
    for (int k = 0; k < kVec<DT>; ++k) acc += weight(it, k);
    vs[it] = acc;
  }
  // Cell (it, wave) totals: lane 63 of each wavefront's inclusive scan.
  float tot[NL];
#pragma unroll
  for (int it = 0; it < NL; ++it) tot[it] = vs[it];
  wave_inclusive_sum_n(tot);
#pragma unroll
  for (int it = 0; it < NL; ++it) tot[it] = lane63(tot[it]);
  if (l == 0) {
#pragma unroll
    for (int it = 0; it < NL; ++it) sh.cell[it * kWaves + w] = tot[it];
  }
  __syncthreads();
  // Every wavefront finds the cell (the same scan gives the same answer).
  const float cv = (l < NL * kWaves) ? sh.cell[l] : 0.0f;
  const float inc = wave_inclusive_sum(cv);
  const float exc = wave_shift_up1(inc);
  const unsigned long long hit =
      __ballot(l < NL * kWaves && exc <= t_in && t_in < inc);
  const int cell = hit ? __ffsll((unsigned long long)hit) - 1 : -1;
  if (cell < 0) {
    if (tid == 0) sh.result = kDrawPastEnd;
  } else if (w == cell % kWaves) {
    const int its = cell / kWaves;
    float v = vs[0];
#pragma unroll
    for (int it = 1; it < NL; ++it)
      if (it == its) v = vs[it];
    const float tc = fmaxf(0.0f, t_in - readlane_f(exc, cell));
    const float inc2 = wave_inclusive_sum(v);
    const float exc2 = wave_shift_up1(inc2);
    const bool mine = exc2 <= tc && tc < inc2;
    const unsigned long long who = __ballot(mine);
    if (!who) {
      if (l == 0) sh.result = kDrawPastEnd;
    } else if (mine && l == __ffsll((unsigned long long)who) - 1) {
      const float tl = tc - exc2;
      u32x4 rv = raw[0];
      float qv[kVec<DT>];
#pragma unroll
      for (int k = 0; k < kVec<DT>; ++k) qv[k] = q.at(0, k);
#pragma unroll
      for (int it = 1; it < NL; ++it)
        if (it == its) {
          rv = raw[it];
#pragma unroll
          for (int k = 0; k < kVec<DT>; ++k) qv[k] = q.at(it, k);
        }
      float run = 0.0f, lfound = NAN, llast = NAN;
      int found = -1, lastp = -1;
#pragma unroll
      for (int k = 0; k < kVec<DT>; ++k) {
        const int i = index(its, k);
        const float lk = elem<DT>(rv, k);
        const float wk = draw_weight<DT, RESIDUAL>(lk, i, excl, m, kk, invS, qv[k], lam);
        run += wk;
        if (wk > 0.0f) {
          lastp = i;
          llast = lk;
        }
        if (found < 0 && run > tl) {
          found = i;
          lfound = lk;
        }
      }
      sh.result = found >= 0 ? found : lastp;
      sh.result_l = found >= 0 ? lfound : llast;
    }
  }
  __syncthreads();
  if (sh.result == kDrawPastEnd) {
    // The target lies past the re-read total (rounding): the last token of
    // positive weight it re-read, found only now, as the common path needs
    // none of it. The weights are the same instructions on the same inputs
    // as above, so the same ones are positive.
    int tlast = -1;
#pragma unroll
    for (int it = 0; it < NL; ++it)
#pragma unroll
      for (int k = 0; k < kVec<DT>; ++k)
        if (weight(it, k) > 0.0f) tlast = max(tlast, index(it, k));
    tlast = wave_max_i(tlast);
    if (l == 0) sh.wlast[w] = tlast;
    __syncthreads();
    if (tid == 0) {
      int clast = sh.wlast[0];
      for (int i = 1; i < kWaves; ++i) clast = max(clast, sh.wlast[i]);
      sh.result = clast;
      sh.result_l = NAN;
    }
    __syncthreads();
  }
  return sh.result;
}

}  // namespace
}  // namespace specsam
