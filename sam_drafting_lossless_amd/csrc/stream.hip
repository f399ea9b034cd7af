// Stream pass of the batched verification: reads every logit row a sequence
// needs once, in 32 KiB chunks, and leaves one partial per (row, chunk).
//
// Method ([P2] m.nxbn.cn guide §2.2; [P3] gogongxt notes "贪婪采样",
// "拒绝采样"): row j of sequence b is needed iff j <= draft_len[b] (rows past
// the drafts are never read). At T = 0 a partial is (max, lowest index of the
// max, NaN flag); at T > 0 it is the online (max m, sum of exp2((l - m) *
// log2e / T)) plus the logit of the draft token x_j when x_j falls in the
// chunk. The finish pass combines them. When the request truncates its
// target (top-k / top-p), each chunk of a row at T > 0 also leaves a window
// histogram of its logits and copies the logits of a band of its bins (the
// ones that probably hold the row's threshold) to its candidate segment, for
// the selection kernel (trunc.hip).
//
// Design for gfx950: 256-thread workgroups each hold one chunk in registers
// (8 non-temporal 16-byte loads in flight per lane, each wavefront load one
// contiguous 1 KiB request) and write one 16-byte partial per row: nothing
// but loads, arithmetic and one store. The grid is (sequence, row lane,
// chunk): lane q of a sequence streams its chunk of rows q, q + G, q + 2G,
// ... up to the sequence's draft length. Launches whose row 0 alone gives
// fewer than 4096 workgroups (and draft trees) take G = K + 1, a workgroup
// per needed (row, chunk); larger ones take G = 2 for K <= 3 and 4 above,
// so that a sequence with no drafts leaves few idle workgroups per chunk
// (they read its draft length and leave) while drafted rows still spread
// over several workgroups.
#include <algorithm>
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

// LDS of a truncated row's chunk: its window histogram (and one spare word
// per lane, which takes the adds of tokens outside the window, so that every
// element adds without a branch), each wavefront's run of band logits (and a
// spare slot per lane for the writes of tokens outside the band), the band
// and the runs' lengths.
struct TrShared {
  unsigned long long hs[kHistBins + kWave];
  float run[kWaves][kSegCap + kWave];
  int band[2];
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
// window too; lo > hi: none):
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
// relative to its max; nfin: its finite count; k, tp: the row's top_k (0:
// none) and top_p.
__device__ __forceinline__ int2 choose_band(const unsigned long long* hs, float total,
                                            int nfin, int k, float tp, int V, int cap) {
  const int l = threadIdx.x % kWave;
  // Cumulative counts (c*) and weights (m*) from the top through each of
  // the lane's four bins.
  const unsigned long long w0 = hs[4 * l], w1 = hs[4 * l + 1], w2 = hs[4 * l + 2],
                           w3 = hs[4 * l + 3];
  float c0 = (float)(unsigned)(w0 >> 48), c1 = (float)(unsigned)(w1 >> 48),
        c2 = (float)(unsigned)(w2 >> 48), c3 = (float)(unsigned)(w3 >> 48);
  float m0 = (float)(w0 & kMassMask), m1 = (float)(w1 & kMassMask),
        m2 = (float)(w2 & kMassMask), m3 = (float)(w3 & kMassMask);
  const float lc = (c0 + c1) + (c2 + c3);  // exact: < 2^24
  const float lm = ((m0 + m1) + (m2 + m3)) * (1.0f / kFixScale);
  c0 += wave_inclusive_sum(lc) - lc;
  c1 += c0;
  c2 += c1;
  c3 += c2;
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
  return int2{lo, hi};
}

// Reduces one loaded chunk of row j of sequence b into its partial. `raw`
// holds the chunk; `mid` runs once every element has been consumed (after
// the last pass that reads `raw`), before the workgroup reduction. With TR, a
// truncated row also leaves its chunk's window histogram and band (ts is the
// LDS for them). Ends with a barrier, so `red` and `ts` may be reused at once.

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
    float s = 0.0f;
    int nfin = 0;  // wavefront-uniform
#pragma unroll
    for (int it = 0; it < kLoads; ++it)
#pragma unroll
      for (int k = 0; k < kVec<DT>; ++k) {
        const float v = elem<DT>(raw[it], k);
        const float wv = fast_exp2(fmaf(v, kk, -bkk));
        s += wv;
        keep_here(s);
        // -inf (probability 0) and NaN are not counted. The masks are
        // ballots of the compares, combined on the scalar unit, so the
        // element takes no branch.
        const bool fin = v > kNegInf;
        nfin += __popcll(ballot_mask(fin));
        keep_here_uniform(nfin);
        const int jb = abs_bin_s(v, ns) - a0;
        const bool inw = fin & ((unsigned)jb < (unsigned)kHistBins);
        atomicAdd(&ts->hs[inw ? jb : kHistBins + l],
                  kCountOne | (unsigned long long)(unsigned)(wv * kFixScale));
      }
    s = wave_sum(s);
    const float nf = (float)nfin;  // exact: < 2^24
    __syncthreads();  // every lane has read red[].x; the histogram is complete
    if (l == 0) {
      red[w].y = s;
      red[w].z = nf;
    }
    __syncthreads();
    float ps = 0.0f, nft = 0.0f;
    for (int i = 0; i < kWaves; ++i) {
      ps += red[i].y;
      nft += red[i].z;
    }
    const int64_t hc = row * nc + c;
    a.hist[hc * kHistBins + tid] = ts->hs[tid];
    if (w == 0) {
      const int2 bd = choose_band(ts->hs, ps, (int)nft, tk, tp, a.V, a.segcap);
      if (l == 0) {
        ts->band[0] = bd.x;
        ts->band[1] = bd.y;
      }
    }
    __syncthreads();
    const int blo = ts->band[0], bhi = ts->band[1];
    // (the bins and weights are recomputed: kept from the histogram pass,
    // they would hold 64 more registers across the barriers)
#pragma unroll
    for (int it = 0; it < kLoads; ++it) keep_here(raw[it]);
    // Band and above-band tests on the product t = l * ns (see band_t): the
    // band holds the tokens with t in [lo_f, hi_f), the tokens above it
    // have t < lo_f. The weight above the band is summed only when the band
    // does not start at the chunk max (top-p alone). No branch per element:
    // a token outside the band writes its lane's spare slot.
    const float lo_f = (float)(a0 + blo);
    const float hi_f = bhi >= kRestBin ? INFINITY : (float)(a0 + bhi + 1);
    float above = 0.0f;
    int n = 0;  // wavefront-uniform
    float* run = ts->run[w];
    auto band_pass = [&](auto with_above) {
#pragma unroll
      for (int it = 0; it < kLoads; ++it)
#pragma unroll
        for (int k = 0; k < kVec<DT>; ++k) {
          const float v = elem<DT>(raw[it], k);
          const float t = v * ns;
          const bool lo = t >= lo_f;
          if constexpr (decltype(with_above)::value) {
            const float wv = fast_exp2(fmaf(v, kk, -bkk));
            above += lo ? 0.0f : wv;
            keep_here(above);
          }
          const bool inb = lo & (t < hi_f);
          const unsigned long long hit = ballot_mask(inb);
          const int p = n + lanes_below(hit);
          run[(inb & (p < kSegCap)) ? p : kSegCap + l] = v;
          n += __popcll(hit);
        }
    };
    if (blo > 0)
      band_pass(std::true_type{});
    else
      band_pass(std::false_type{});
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
    // A band whose tokens do not fit (possible only for non-finite logits,
    // which the histogram does not count) is reported as none.
    const bool ok = blo <= bhi && tot <= a.segcap;
    if (ok) {
      float* out = a.cand + hc * a.segcap + wbase;
      for (int p = l; p < n; p += kWave) out[p] = run[p];
    }
    if (tid == 0) {
      a.hhdr[hc] = i32x4{a0, (int)nft, ok ? (blo | (bhi << 16)) : kNoBand, ok ? tot : 0};
      a.tpart[hc] = ab;
    }
    part = f32x4{pm, ps, hasx ? red[kWaves].x : lx, 0.0f};
    }
  } else {
    // Online (max, sum exp2) folded one 16-byte vector at a time, in the
    // order the loads return, so only the raw vectors stay live. The draft
    // token's logit is taken in a copy of the loop that only the chunk
    // holding it runs (hasx is the same for the whole workgroup).
    float m = kNegInf, s = 0.0f;
    auto fold = [&](auto take_x) {
#pragma unroll
      for (int it = 0; it < kLoads; ++it) {
        float vm = kNegInf;
#pragma unroll
        for (int k = 0; k < kVec<DT>; ++k) vm = fmaxf(vm, elem<DT>(raw[it], k));
        const float mn = fmaxf(m, vm);
        const float base = (mn == kNegInf) ? 0.0f : mn;
        float t = s * fast_exp2((m - base) * kk);
#pragma unroll
        for (int k = 0; k < kVec<DT>; ++k) {
          const float v = elem<DT>(raw[it], k);
          t += fast_exp2((v - base) * kk);
          if constexpr (decltype(take_x)::value) xv = (ex == it * kVec<DT> + k) ? v : xv;
        }
        s = t;
        m = mn;
      }
    };
    if (hasx)
      fold(std::true_type{});
    else
      fold(std::false_type{});
    if (ex >= 0) red[kWaves].x = xv;  // read after the reduction's barrier
    mid();
    wave_lse(m, s, kk);
    if (l == 0) red[w] = f32x4{m, s, 0.0f, 0.0f};
    __syncthreads();
    float pm = red[0].x, ps = red[0].y;
    for (int i = 1; i < kWaves; ++i) lse_merge(pm, ps, red[i].x, red[i].y, kk);
    part = f32x4{pm, ps, hasx ? red[kWaves].x : lx, 0.0f};
  }
  if (tid == 0) a.partials[row * nc + c] = part;
  __syncthreads();  // red[] is reused by the next row
}

struct NoMid {
  __device__ void operator()() const {}
};

// Occupancy hint, for the histogram variant on the 16-byte load path only:
// 5 (fp32) or 3 (bf16) waves per SIMD. Under a hint of 6 the fp32 code
// spills a few registers to scratch, and the reloads, each a memory round
// trip, cost more than the extra wavefront gains (B = 256, V = 151936, no
// drafts, top-p: 56.4 us at 5 against 63.0 at 6). The plain variant takes
// none: the compiler then schedules it with 90
// registers (5 waves per SIMD), against 61 (8 waves) under a hint of 6, and
// that code streams faster once many rows are needed (B = 256, V = 151936,
// K = 3, every draft full: 94.0 us against 97.5, equal with no drafts). The
// element-wise path takes none either: it would spill under one.
template <int DT, bool TR>
constexpr int kStreamWaves = (DT == SS_DTYPE_F32) ? 5 : 3;

// Row lanes G (see the file comment). Measured per launch at B = 256,
// V = 151936, fp32, K = 3 (events around 8 back-to-back launches, one box):
//   draft lengths        G = 2    G = 4    kernel replaced (*)
//   all 0 (256 rows)     27.4     32.3     27.9 us
//   c3-like (277 rows)   29.4     33.2     30.3
//   uniform 0..3         62.0     61.9     67.5
//   all 3 (1024 rows)    94.0     90.1    103.1
// (*) one workgroup per (sequence, chunk) of row 0, the chunks of rows
// 1..d dealt round-robin to the same workgroups: each took its extra items
// one after another, and every gap between them left its CU with fewer
// loads in flight. At K = 16 two lanes serialise too many rows (a c3-like
// mix took 48.9 us against 39.6 with four lanes).
constexpr int64_t kRow0Fill = 4096;  // row-0 workgroups that fill the chip
inline int row_lanes(int B, int K, int nchunks) {
  if ((int64_t)B * nchunks < kRow0Fill) return K + 1;
  return std::min(K + 1, K <= 3 ? 2 : 4);
}

// Grid: (sequence b, row lane q, chunk c), c fastest. Row 0, which every
// valid sequence needs, is requested before the sequence's parameters
// return; lanes q >= 1 first learn the draft length.
template <int DT, bool VP, bool TR>
__global__ __launch_bounds__(kThreads, ((VP && TR) ? kStreamWaves<DT, TR> : 1)) void
spec_stream_kernel(Args a) {
  __shared__ f32x4 red[kWaves + 1];
  __shared__ TrLds<TR> tl;
  TrShared* ts = nullptr;
  if constexpr (TR) ts = &tl.s;
  const int tid = threadIdx.x;
  const int R = a.K + 1, nc = a.nchunks, G = a.ngroups;
  const int c = blockIdx.x % nc;
  const int bq = blockIdx.x / nc;
  const int b = bq / G, q = bq - b * G;
  const int cstart = c * kChunk<DT>;
  u32x4 raw[kLoads];
  if (q == 0)
    load_chunk<DT, VP>(a.logits + (int64_t)b * R * a.V * Dt<DT>::kBytes, cstart,
                       a.V, tid, raw);
  int x = draft_token(a, b, q);
  int d;
  float T;
  const int st = seq_check(a, b, &d, &T);  // reported by finalize
  if (st) return;
  for (int j = q; j <= d; j += G) {
    if (j != 0)
      load_chunk<DT, VP>(a.logits + ((int64_t)b * R + j) * a.V * Dt<DT>::kBytes,
                         cstart, a.V, tid, raw);
    if (j != q) x = draft_token(a, b, j);
    stream_row<DT, VP, TR, true>(a, b, j, d, T, c, x, raw, red, ts, NoMid{});
  }
}

// Draft trees: a tree's nodes usually all need their rows, so every
// (sequence, node, chunk) gets a workgroup (G = K + 1).
inline bool tree_rows(const Args& a) { return a.dl_status == SS_ST_TREE; }

template <int DT, bool VP, bool TR>
int launch_stream_t(const Args& a, hipStream_t s) {
  const int64_t grid = (int64_t)a.B * a.nchunks * a.ngroups;
  if (grid > INT_MAX) return set_error(SS_EINVAL, "spec_stream: grid too large");
  hipLaunchKernelGGL((spec_stream_kernel<DT, VP, TR>), dim3((unsigned)grid),
                     dim3(kThreads), 0, s, a);
  return check_launch("spec_stream");
}

template <int DT, bool VP>
int launch_stream_tr(const Args& a, hipStream_t s) {
  return a.hist ? launch_stream_t<DT, VP, true>(a, s)
                : launch_stream_t<DT, VP, false>(a, s);
}

}  // namespace

int launch_stream(Args a, bool f32, bool vp, hipStream_t s) {
  a.ngroups = tree_rows(a) ? a.K + 1 : row_lanes(a.B, a.K, a.nchunks);
  return f32 ? (vp ? launch_stream_tr<SS_DTYPE_F32, true>(a, s)
                   : launch_stream_tr<SS_DTYPE_F32, false>(a, s))
             : (vp ? launch_stream_tr<SS_DTYPE_BF16, true>(a, s)
                   : launch_stream_tr<SS_DTYPE_BF16, false>(a, s));
}

}  // namespace specsam
