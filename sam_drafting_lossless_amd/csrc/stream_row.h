// The stream pass's per-(row, chunk) work, shared by the stream kernel
// (stream.hip) and the small-launch fused step (verify.hip): reduce one
// loaded chunk of a row into its partial, and, for a truncated row, its
// window histogram and band segment.
#pragma once

#include <type_traits>

#include "verify_common.h"

namespace specsam {
namespace {

// ---------------------------------------------------------------------------
// stream: one partial per (row, chunk).
// ---------------------------------------------------------------------------

// The draft token of row j (j < K), or -1; requested with the row's chunk.
__device__ __forceinline__ int draft_token(const Args& a, int b, int j) {
  return (a.draft && j < a.K) ? a.draft[(int64_t)b * a.K + j] : -1;
}

// LDS of a truncated row's chunk: its window histogram, then one word per
// lane that takes the adds of its finite tokens below the window and one
// that takes those of its -inf and NaN tokens (so that every element adds
// without a branch, and the finite count is the sum of the first two
// parts); each wavefront's run of band logits (with room for one more
// ballot's worth past the segment), the band with its logit bounds, and the
// runs' lengths.
struct TrShared {
  unsigned long long hs[kHistBins + 2 * kWave];
  float run[kWaves][kSegCap + kWave];
  int band[4];
  float vb[2];
  float above;  // weight above the band, from the masses (see kFixAboveBins)
  int cnt[kWaves];
};
template <bool TR>
struct TrLds {
  TrShared s;
};
template <>
struct TrLds<false> {
  char s;
};

// (wavefront 0) First bin whose cumulative value reaches t, from the
// lane's cumulative values through its bins 4l .. 4l+3 (nondecreasing over
// the bins); kRestBin if none does.
__device__ __forceinline__ int first_bin(float c0, float c1, float c2, float c3, float t) {
  const unsigned long long hit = __ballot(c3 >= t);
  if (!hit) return kRestBin;
  const int L = __ffsll((unsigned long long)hit) - 1;
  const int q = c0 >= t ? 0 : c1 >= t ? 1 : c2 >= t ? 2 : 3;
  return 4 * L + __builtin_amdgcn_readlane(q, L);
}

// (wavefront 0) The band [lo, hi] of the chunk's window bins whose logits go
// to its candidate segment (hi = kRestBin: every bin from lo down, past the
// window too; lo > hi: none), and the chunk's finite count:
//   top-k: from the chunk max down to the bin where the chunk's own count
//     reaches k. The row's k-th largest logit is at least the chunk's, so
//     the row's threshold range lies within (top-p then works inside what
//     top-k kept);
//   top-p alone: kBandHalf bins either side of the bin where the chunk's
//     cumulative weight reaches top_p of its total. The row's threshold is
//     found near it when the chunk's logits are distributed like the row's.
// The band is narrowed until its tokens fit the segment. The selection
// re-reads a chunk whose band misses the row's range, so the band only
// decides how fast, never what is selected. total: the chunk's weight sum
// relative to its max; k, tp: the row's top_k (0: none) and top_p.
__device__ __forceinline__ int3 choose_band(const unsigned long long* hs, float total, int k,
                                            float tp, int V, int cap) {
  const int l = threadIdx.x % kWave;
  // Cumulative counts (c*) and weights (m*) from the top through each of
  // the lane's four bins.
  const unsigned long long w0 = hs[4 * l], w1 = hs[4 * l + 1], w2 = hs[4 * l + 2],
                           w3 = hs[4 * l + 3], wb = hs[kHistBins + l];
  const int n0 = (int)(w0 >> 48), n1 = (int)(w1 >> 48), n2 = (int)(w2 >> 48),
            n3 = (int)(w3 >> 48);
  float m0 = (float)(w0 & kMassMask), m1 = (float)(w1 & kMassMask),
        m2 = (float)(w2 & kMassMask), m3 = (float)(w3 & kMassMask);
  const int lc = (n0 + n1) + (n2 + n3);
  const float lm = ((m0 + m1) + (m2 + m3)) * (1.0f / kFixScale);
  // One scan carries the window counts (low 16 bits) and the counts below
  // the window (high bits); a chunk has at most 16,384 tokens.
  const int pk = wave_scan(lc | ((int)(wb >> 48) << 16), 0, [](int x, int y) { return x + y; });
  const int tot = lane63(pk);
  const int nfin = (tot & 0xffff) + (tot >> 16);
  float c0 = (float)(((pk & 0xffff) - lc) + n0);  // exact: < 2^24
  float c1 = c0 + (float)n1, c2 = c1 + (float)n2, c3 = c2 + (float)n3;
  // Tokens in bins 0..i (i < 0: none; i = kRestBin: every finite token).
  auto count_through = [&](int i) {
    if (i < 0) return 0;
    if (i >= kHistBins) return nfin;
    const int q = i & 3;
    const float v = q == 0 ? c0 : q == 1 ? c1 : q == 2 ? c2 : c3;
    return (int)__int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), i >> 2));
  };
  int lo = 1, hi = 0;
  if (k >= 1 && k < V) {
    lo = 0;
    hi = first_bin(c0, c1, c2, c3, (float)k);
    if (count_through(hi) > cap) {
      hi = first_bin(c0, c1, c2, c3, (float)(cap + 1)) - 1;  // the top bins that fit
      if (hi < 0) lo = 1;
    }
  } else {
    m0 = m0 * (1.0f / kFixScale) + (wave_inclusive_sum(lm) - lm);
    m1 = m0 + m1 * (1.0f / kFixScale);
    m2 = m1 + m2 * (1.0f / kFixScale);
    m3 = m2 + m3 * (1.0f / kFixScale);
    const int bp = first_bin(m0, m1, m2, m3, tp * total);
    for (int h = kBandHalf; h >= 0; --h) {
      const int l0 = max(0, bp - h);
      const int h0 = bp + h >= kHistBins ? kRestBin : bp + h;
      if (count_through(h0) - count_through(l0 - 1) <= cap) {
        lo = l0;
        hi = h0;
        break;
      }
    }
  }
  return int3{lo, hi, nfin};
}

// Reduces one loaded chunk of row j of sequence b into its partial. `raw`
// holds the chunk; `mid` runs once every element has been consumed (after
// the last pass that reads `raw`), before the workgroup reduction. With TR, a
// truncated row also leaves its chunk's window histogram and band (ts is the
// LDS for them). `red` holds 2 * kWaves + 1 entries. Ends with a barrier, so
// `red` and `ts` may be reused at once.

// x is the draft token of row j (or -1), requested with the chunk. XREG:
// the lane holding its logit takes it with a select as the fold consumes
// that element (no load waited for out of order, two registers); else
// thread 0 loads the logit. The stream kernel takes the first.
template <int DT, bool VP, bool TR, bool XREG, typename Mid>
__device__ __forceinline__ void stream_row(const Args& a, int b, int j, int d,
                                           float T, int c, int x,
                                           u32x4 (&raw)[kLoads], f32x4* red,
                                           TrShared* ts, Mid mid) {
  const int tid = threadIdx.x, w = tid / kWave, l = tid % kWave;
  const int R = a.K + 1, nc = a.nchunks;
  const int cstart = c * kChunk<DT>;
  const int64_t row = (int64_t)b * R + j;
  const bool greedy = (T == 0.0f);
  const float kk = greedy ? 0.0f : kLog2e / T;
  // The logit of the draft token x (row j < d), when it lies in this chunk:
  // loaded by thread 0 into lx, or (XREG) left by the lane holding it in the
  // slot after the reduction slots, read after the reduction's barrier.
  float lx = 0.0f;
  if constexpr (!XREG) {
    if (!greedy && j < d && tid == 0 && a.draft) {
      const int xl = a.draft[(int64_t)b * a.K + j];
      if (xl >= cstart && xl < cstart + kChunk<DT> && xl < a.V)
        lx = load_one<DT>(a.logits + row * a.V * Dt<DT>::kBytes, xl);
    }
  }
  const bool hasx = XREG && !greedy && j < d && x >= cstart && x < cstart + kChunk<DT> &&
                    x < a.V;
  // (XREG) Position ex of x's logit among this lane's elements (it * kVec +
  // k), -1 in every other lane.
  int ex = -1;
  if (hasx) {
    const int o = x - cstart;
    const int itx = o / (kThreads * kVec<DT>);
    const int rem = o - itx * (kThreads * kVec<DT>);
    if (rem / kVec<DT> == tid) ex = itx * kVec<DT> + rem % kVec<DT>;
  }
  float xv = 0.0f;
  f32x4 part;
  if (greedy) {
    // Argmax with the lowest index on ties; position within the lane's
    // elements (it*kVec + k) is a compile-time constant per element, the row
    // index is formed once at the end. Alongside, the online sum of
    // exp(l - max) at temperature 1 (for the log-probabilities of emitted
    // tokens); a NaN anywhere in the chunk makes the sum NaN.
    float bv = kNegInf, s = 0.0f;
    int bp = -1;
#pragma unroll
    for (int it = 0; it < kLoads; ++it)
#pragma unroll
      for (int k = 0; k < kVec<DT>; ++k) {
        const float v = elem<DT>(raw[it], k);
        if (v > bv) {
          bv = v;
          bp = it * kVec<DT> + k;
        }
      }
    float m = kNegInf;
#pragma unroll
    for (int it = 0; it < kLoads; ++it) {
      float vm = kNegInf;
#pragma unroll
      for (int k = 0; k < kVec<DT>; ++k) vm = fmaxf(vm, elem<DT>(raw[it], k));
      const float mn = fmaxf(m, vm);
      const float base = (mn == kNegInf) ? 0.0f : mn;
      float t = s * fast_exp2((m - base) * kLog2e);
#pragma unroll
      for (int k = 0; k < kVec<DT>; ++k)
        t += fast_exp2((elem<DT>(raw[it], k) - base) * kLog2e);
      s = t;
      m = mn;
    }
    mid();
    int bi = bp < 0 ? INT_MAX
                    : elem_index<DT, VP>(cstart, tid, bp / kVec<DT>, bp % kVec<DT>);
    wave_argmax(bv, bi);
    wave_lse(m, s, kLog2e);
    if (l == 0) red[w] = f32x4{bv, s, m, __int_as_float(bi)};
    __syncthreads();
    float pv = red[0].x, pm = red[0].z, ps = red[0].y;
    int pi = __float_as_int(red[0].w);
    for (int i = 1; i < kWaves; ++i) {
      argmax_merge(pv, pi, red[i].x, __float_as_int(red[i].w));
      lse_merge(pm, ps, red[i].z, red[i].y, kLog2e);
    }
    // The sum is relative to the chunk max pm, which equals pv except when
    // the chunk holds NaN (then the sum is NaN and the row is reported).
    part = f32x4{pv, ps, 0.0f, __int_as_float(pi)};
  } else if (TR && trunc_active(a, b, T)) {
    // Truncated row: the chunk max first; then one pass that adds each
    // element's weight exp2((l - max) * log2e / T) to the sum and to the
    // chunk's window histogram (see kHistBins): count and fixed-point weight
    // in one 64-bit word per bin, the bin on the row's shared grid. The
    // chunk's finite count goes to its header (the selection's totals come
    // from the headers and the partials, so nothing below the window is
    // kept). Then the band (choose_band) and a last pass that copies the
    // band's logits to the chunk's segment, in (wavefront, element, lane)
    // order, and sums the weight of the tokens above the band.
    if constexpr (TR) {
    const int tk = a.top_k ? a.top_k[b] : 0;
    const float tp = a.top_p ? a.top_p[b] : 1.0f;
    // (the draft token's logit is taken in a copy of the loop that only the
    // chunk holding it runs: hasx is the same for the whole workgroup)
    float vm = kNegInf;
    if (hasx) {
#pragma unroll
      for (int it = 0; it < kLoads; ++it)
#pragma unroll
        for (int k = 0; k < kVec<DT>; ++k) {
          const float v = elem<DT>(raw[it], k);
          vm = fmaxf(vm, v);
          xv = (ex == it * kVec<DT> + k) ? v : xv;
        }
      if (ex >= 0) red[kWaves].x = xv;  // read after the barrier below
    } else {
#pragma unroll
      for (int it = 0; it < kLoads; ++it)
#pragma unroll
        for (int k = 0; k < kVec<DT>; ++k) vm = fmaxf(vm, elem<DT>(raw[it], k));
    }
    vm = wave_max(vm);
    ts->hs[tid] = 0;
    if (tid < 2 * kWave) ts->hs[kHistBins + tid] = 0;
    if (l == 0) red[w] = f32x4{vm, 0.0f, 0.0f, 0.0f};
    __syncthreads();
    float pm = red[0].x;
    for (int i = 1; i < kWaves; ++i) pm = fmaxf(pm, red[i].x);
    const float base = (pm == kNegInf) ? 0.0f : pm;
    const float ns = bin_scale(kk);
    const int a0 = abs_bin_s(pm, ns);
    // (bf16: the elements are re-extracted from their packed registers;
    // converted once for every pass, the chunk would be held as 64 floats)
    if constexpr (DT != SS_DTYPE_F32) {
#pragma unroll
      for (int it = 0; it < kLoads; ++it) keep_here(raw[it]);
    }
    // (a truncated row's weights are exp2(l * kk - base * kk), one fma and
    // one exp per element; its partial comes only from this branch)
    const float bkk = base * kk;
    // A token outside the window adds to its lane's word below the window
    // (finite) or to its non-finite word: one unsigned min and one select.
    const unsigned below = (unsigned)(kHistBins + l);
    const unsigned nonfin = (unsigned)(kHistBins + kWave + l);
    float s = 0.0f;
#pragma unroll
    for (int it = 0; it < kLoads; ++it)
#pragma unroll
      for (int k = 0; k < kVec<DT>; ++k) {
        const float v = elem<DT>(raw[it], k);
        const float wv = fast_exp2(fmaf(v, kk, -bkk));
        s += wv;
        keep_here(s);
        const unsigned jb = min((unsigned)(abs_bin_s(v, ns) - a0), below);
        atomicAdd(&ts->hs[v > kNegInf ? jb : nonfin],
                  kCountOne | (unsigned long long)(unsigned)fmaf(wv, kFixScale, 0.5f));
      }
    s = wave_sum(s);
    if (l == 0) red[w].y = s;  // (red[].x, read above, stays)
    __syncthreads();            // the histogram is complete
    float ps = 0.0f;
    for (int i = 0; i < kWaves; ++i) ps += red[i].y;
    const int64_t hc = row * nc + c;
    a.hist[hc * kHistBins + tid] = ts->hs[tid];
    if (w == 0) {
      // The band, and its bounds as logits: t = l * ns lies in [lo_f, hi_f)
      // exactly when vb[0] <= l <= vb[1], and below lo_f (above the band)
      // exactly when l > vb[1] (logit_upto). Bounds that do not settle
      // leave the chunk without a band.
      const int3 bd = choose_band(ts->hs, ps, tk, tp, a.V, a.segcap);
      int lo = bd.x, hi = bd.y;
      float vtop = 0.0f, vex = 0.0f;
      if (lo <= hi) {
        const float lo_f = (float)(a0 + lo);
        const float hi_f = hi >= kRestBin ? INFINITY : (float)(a0 + hi + 1);
        const bool top_ok = logit_upto(lo_f, ns, &vtop);
        const bool bot_ok = logit_upto(hi_f, ns, &vex);
        if (!(top_ok && bot_ok)) {
          lo = 1;
          hi = 0;
        }
      }
      // The weight above a band near the chunk max: the masses of the bins
      // above it (each below 2^46, exact in double; the sum below 2^54).
      float abf = 0.0f;
      if (lo > 0 && lo <= hi && lo <= kFixAboveBins) {
        double mb = 0.0;
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (4 * l + q < lo) mb += (double)(ts->hs[4 * l + q] & kMassMask);
        abf = (float)(wave_sum_d(mb) * (1.0 / (double)kFixScale));
      }
      if (l == 0) {
        ts->band[0] = lo;
        ts->band[1] = hi;
        ts->band[2] = bd.z;
        ts->vb[0] = float_step(vex, 1);
        ts->vb[1] = vtop;
        ts->above = abf;
      }
    }
    __syncthreads();
    const int blo = ts->band[0], bhi = ts->band[1];
    const float vbot = ts->vb[0], vtop = ts->vb[1];
    // (the weights are recomputed: kept from the histogram pass, they would
    // hold 32 more registers across the barriers)
#pragma unroll
    for (int it = 0; it < kLoads; ++it) keep_here(raw[it]);
    // The band's logits go to the wavefront's run in (element, lane) order:
    // a ballot, the lane's rank among the hits, an exec-masked LDS store. n
    // counts every hit; positions stop at kSegCap, so that a run that
    // overflows (the band is then reported as none) stays inside its room.
    // The weight above the band is summed here only for a band that starts
    // deeper than kFixAboveBins below the chunk max (top-p alone); nearer
    // ones took it from the histogram.
    float above = 0.0f;
    int n = 0, np = 0;  // wavefront-uniform
    float* run = ts->run[w];
    auto band_pass = [&](auto with_above) {
#pragma unroll
      for (int it = 0; it < kLoads; ++it)
#pragma unroll
        for (int k = 0; k < kVec<DT>; ++k) {
          const float v = elem<DT>(raw[it], k);
          if constexpr (decltype(with_above)::value) {
            const float wv = fast_exp2(fmaf(v, kk, -bkk));
            above += (v > vtop) ? wv : 0.0f;
            keep_here(above);
          }
          const bool inb = __builtin_amdgcn_fmed3f(v, vbot, vtop) == v;
          const unsigned long long hit = ballot_mask(inb);
          if (inb) run[np + lanes_below(hit)] = v;
          n += __popcll(hit);
          np = min(n, kSegCap);
        }
    };
    const bool fix_above = blo <= kFixAboveBins;  // (or no weight above: blo = 0)
    if (blo > bhi) {
    } else if (!fix_above) {
      band_pass(std::true_type{});
    } else {
      band_pass(std::false_type{});
    }
    mid();  // the band pass was the last to read `raw`
    above = wave_sum(above);
    if (l == 0) {
      ts->cnt[w] = n;
      red[w].w = above;
    }
    __syncthreads();
    int wbase = 0, tot = 0;
    float ab = 0.0f;
    for (int i = 0; i < kWaves; ++i) {
      wbase += (i < w) ? ts->cnt[i] : 0;
      tot += ts->cnt[i];
      ab += red[i].w;
    }
    if (fix_above) ab = ts->above;
    // A band whose tokens do not fit (possible only for non-finite logits,
    // which the histogram does not count) is reported as none.
    const bool ok = blo <= bhi && tot <= a.segcap;
    if (ok) {
      float* out = a.cand + hc * a.segcap + wbase;
      for (int p = l; p < n; p += kWave) out[p] = run[p];
    }
    if (tid == 0) {
      a.hhdr[hc] = i32x4{a0, ts->band[2], ok ? (blo | (bhi << 16)) : kNoBand, ok ? tot : 0};
      a.tpart[hc] = ab;
    }
    part = f32x4{pm, ps, hasx ? red[kWaves].x : lx, 0.0f};
    }
  } else {
    // Two passes over the registers: the chunk max M, then each element's
    // weight exp2((l - M) * log2e / T), summed per quarter of the chunk
    // (loads 2q and 2q + 1: a contiguous quarter of its tokens). The
    // partial's sum is the quarters' (s0 + s1) + (s2 + s3); the quarter sums
    // let a draw from this chunk re-read one quarter. The draft token's
    // logit is taken in a copy of the max loop that only the chunk holding
    // it runs (hasx is the same for the whole workgroup).
    static_assert(kLoads == 8 && kWaves == 4, "quarters of two loads");
    float vm = kNegInf;
    auto max_pass = [&](auto take_x) {
#pragma unroll
      for (int it = 0; it < kLoads; ++it)
#pragma unroll
        for (int k = 0; k < kVec<DT>; ++k) {
          const float v = elem<DT>(raw[it], k);
          vm = fmaxf(vm, v);
          if constexpr (decltype(take_x)::value) xv = (ex == it * kVec<DT> + k) ? v : xv;
        }
    };
    if (hasx)
      max_pass(std::true_type{});
    else
      max_pass(std::false_type{});
    if (ex >= 0) red[kWaves].x = xv;  // read after the barriers below
    vm = wave_max(vm);
    if (l == 0) red[w].x = vm;
    __syncthreads();
    float pm = red[0].x;
    for (int i = 1; i < kWaves; ++i) pm = fmaxf(pm, red[i].x);
    const float base = (pm == kNegInf) ? 0.0f : pm;
    float sq[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float t = 0.0f;
#pragma unroll
      for (int it = 2 * q; it < 2 * q + 2; ++it)
#pragma unroll
        for (int k = 0; k < kVec<DT>; ++k) t += fast_exp2((elem<DT>(raw[it], k) - base) * kk);
      sq[q] = t;
    }
    mid();
    wave_inclusive_sum_n(sq);
    if (l == kWave - 1) red[kWaves + 1 + w] = f32x4{sq[0], sq[1], sq[2], sq[3]};
    __syncthreads();
    f32x4 qs = red[kWaves + 1];
    for (int i = 1; i < kWaves; ++i) {
      const f32x4 o = red[kWaves + 1 + i];
      qs = f32x4{qs.x + o.x, qs.y + o.y, qs.z + o.z, qs.w + o.w};
    }
    part = f32x4{pm, (qs.x + qs.y) + (qs.z + qs.w), hasx ? red[kWaves].x : lx, 0.0f};
    if (tid == 0 && a.wparts) a.wparts[row * nc + c] = qs;
  }
  if (tid == 0) a.partials[row * nc + c] = part;
  __syncthreads();  // red[] is reused by the next row
}

struct NoMid {
  __device__ void operator()() const {}
};

}  // namespace
}  // namespace specsam
