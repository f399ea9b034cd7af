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
// histogram of its logits for the truncation passes (trunc.hip).
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

#include "verify_common.h"

namespace specsam {
namespace {

// ---------------------------------------------------------------------------
// stream: one partial per (row, chunk).
// ---------------------------------------------------------------------------

// Reduces one loaded chunk of row j of sequence b into its partial. `raw`
// holds the chunk; `mid` runs once every element has been consumed (after
// the last pass that reads `raw`), before the workgroup reduction. With TR, a
// truncated row also leaves its chunk's window histogram (hs is the LDS
// histogram). Ends with a barrier, so `red` and `hs` may be reused at once.
// The draft token of row j (j < K), or -1; requested with the row's chunk.
__device__ __forceinline__ int draft_token(const Args& a, int b, int j) {
  return (a.draft && j < a.K) ? a.draft[(int64_t)b * a.K + j] : -1;
}

// x is the draft token of row j (or -1), requested with the chunk. XREG:
// the lane holding its logit takes it with a select as the fold consumes
// that element (no load waited for out of order, two registers); else
// thread 0 loads the logit. The stream kernel takes the first.
template <int DT, bool VP, bool TR, bool XREG, typename Mid>
__device__ __forceinline__ void stream_row(const Args& a, int b, int j, int d,
                                           float T, int c, int x,
                                           u32x4 (&raw)[kLoads], f32x4* red,
                                           unsigned long long* hs, Mid mid) {
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
    // Truncated row: the chunk max first, then one pass that adds each
    // element's weight exp2((l - max) * log2e / T) to the sum and to the
    // chunk's window histogram (see kHistBins): count and fixed-point weight
    // in one 64-bit word per bin, the bin on the row's shared grid. The
    // chunk's finite count goes to its header (the plan's totals come from
    // the headers and the partials, so nothing below the window is kept).
    float vm = kNegInf;
#pragma unroll
    for (int it = 0; it < kLoads; ++it)
#pragma unroll
      for (int k = 0; k < kVec<DT>; ++k) {
        const float v = elem<DT>(raw[it], k);
        vm = fmaxf(vm, v);
        xv = (ex == it * kVec<DT> + k) ? v : xv;
      }
    if (ex >= 0) red[kWaves].x = xv;  // read after the barrier below
    vm = wave_max(vm);
    hs[tid] = 0;
    if (l == 0) red[w] = f32x4{vm, 0.0f, 0.0f, 0.0f};
    __syncthreads();
    float pm = red[0].x;
    for (int i = 1; i < kWaves; ++i) pm = fmaxf(pm, red[i].x);
    const float base = (pm == kNegInf) ? 0.0f : pm;
    const int a0 = abs_bin(pm, kk);
    // (bf16: the elements are re-extracted from their packed registers;
    // converted once for both passes, the chunk would be held as 64 floats)
    if constexpr (DT != SS_DTYPE_F32) {
#pragma unroll
      for (int it = 0; it < kLoads; ++it) keep_here(raw[it]);
    }
    float s = 0.0f;
    int nfin = 0;  // wavefront-uniform
#pragma unroll
    for (int it = 0; it < kLoads; ++it)
#pragma unroll
      for (int k = 0; k < kVec<DT>; ++k) {
        const float v = elem<DT>(raw[it], k);
        const float wv = fast_exp2((v - base) * kk);
        s += wv;
        keep_here(s);
        // -inf (probability 0) and NaN are not counted; one condition, so
        // that the element takes a single branch
        const bool fin = v > kNegInf;
        nfin += __popcll(__ballot(fin));
        keep_here_uniform(nfin);
        const int jb = abs_bin(v, kk) - a0;
        if (fin && (unsigned)jb < (unsigned)kHistBins)
          atomicAdd(&hs[jb], kCountOne | (unsigned long long)(unsigned)(wv * kFixScale));
      }
    mid();  // the second pass was the last to read `raw`
    s = wave_sum(s);
    const float nf = (float)nfin;  // exact: < 2^24
    __syncthreads();  // every lane has read red[].x
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
    part = f32x4{pm, ps, hasx ? red[kWaves].x : lx, 0.0f};
    const int64_t hc = row * nc + c;
    a.hist[hc * kHistBins + tid] = hs[tid];
    if (tid == 0) a.hhdr[hc] = i32x4{a0, (int)nft, 0, 0};
  } else {
    // Online (max, sum exp2) folded one 16-byte vector at a time, in the
    // order the loads return, so only the raw vectors stay live.
    float m = kNegInf, s = 0.0f;
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
        xv = (ex == it * kVec<DT> + k) ? v : xv;
      }
      s = t;
      m = mn;
    }
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
// 6 (fp32) or 3 (bf16) waves per SIMD (a tighter bf16 hint spills to
// scratch; LDS limits this variant to 6 workgroups per CU anyway). The
// plain variant takes none: the compiler then schedules it with 90
// registers (5 waves per SIMD), against 61 (8 waves) under a hint of 6, and
// that code streams faster once many rows are needed (B = 256, V = 151936,
// K = 3, every draft full: 94.0 us against 97.5, equal with no drafts). The
// element-wise path takes none either: it would spill under one.
template <int DT, bool TR>
constexpr int kStreamWaves = (DT == SS_DTYPE_F32) ? 6 : 3;

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
  __shared__ unsigned long long hs[TR ? kHistBins : 1];
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
  if (TR && blockIdx.x == 0 && tid == 0) *a.tcount = 0;  // rows the plan lists
  if (st) return;
  for (int j = q; j <= d; j += G) {
    if (j != 0)
      load_chunk<DT, VP>(a.logits + ((int64_t)b * R + j) * a.V * Dt<DT>::kBytes,
                         cstart, a.V, tid, raw);
    if (j != q) x = draft_token(a, b, j);
    stream_row<DT, VP, TR, true>(a, b, j, d, T, c, x, raw, red, hs, NoMid{});
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
