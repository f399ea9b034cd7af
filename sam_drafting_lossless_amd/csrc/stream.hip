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
// but loads, arithmetic and one store. The balanced kernel (batches up to
// 2048 sequences with at least 4096 (sequence, chunk) pairs) gives every
// (sequence, chunk) of row 0 its own workgroup and deals the chunks of rows
// 1..draft_len round-robin to the same workgroups, so that the ones with
// extra work are dispatched first; smaller batches give every (sequence,
// row, chunk) a workgroup, larger ones use a (sequence, row group, chunk)
// grid.
#include <algorithm>

#include "verify_common.h"

namespace specsam {
namespace {

// ---------------------------------------------------------------------------
// stream: one partial per (row, chunk).
// ---------------------------------------------------------------------------

// Reduces one loaded chunk of row j of sequence b into its partial. `raw`
// holds the chunk; `mid` runs once every element has been consumed, before
// the workgroup reduction (the balanced kernel issues its next item's loads
// into `raw` there). With TR, a truncated row also leaves its chunk's window
// histogram (hs is the LDS histogram). Ends with a barrier, so `red` and `hs`
// may be reused at once.
// The draft token of row j (j < K), or -1; requested with the row's chunk.
__device__ __forceinline__ int draft_token(const Args& a, int b, int j) {
  return (a.draft && j < a.K) ? a.draft[(int64_t)b * a.K + j] : -1;
}

// XREG: x (the draft token, or -1) was requested with the chunk, and the
// lane holding its logit takes it from its registers; else thread 0 loads x
// and then its logit. The grid kernel, whose workgroups stream one row each,
// takes the first (no dependent loads after the chunk's); the balanced
// kernel the second (measured: as fast there, and it keeps the bf16
// variant's register count, and so its occupancy, lower).
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
  if (hasx) {
    const int o = x - cstart;
    const int itx = o / (kThreads * kVec<DT>);
    const int rem = o - itx * (kThreads * kVec<DT>);
    if (rem / kVec<DT> == tid) {
      // its 32-bit word among the lane's 8 x 4, then the element in it
      const int kx = rem % kVec<DT>;
      const int wx = kx / (kVec<DT> / 4);
      unsigned wv = 0;
#pragma unroll
      for (int it = 0; it < kLoads; ++it)
#pragma unroll
        for (int q = 0; q < 4; ++q)
          if (it == itx && q == wx) wv = raw[it][q];
      // (a bf16 word holds two elements: kx & 1 picks the half)
      const u32x4 one = u32x4{wv, wv, wv, wv};
      red[kWaves].x = elem<DT>(one, DT == SS_DTYPE_F32 ? 0 : (kx & 1));
    }
  }
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
      for (int k = 0; k < kVec<DT>; ++k) vm = fmaxf(vm, elem<DT>(raw[it], k));
    mid();
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
      for (int k = 0; k < kVec<DT>; ++k)
        t += fast_exp2((elem<DT>(raw[it], k) - base) * kk);
      s = t;
      m = mn;
    }
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

// Occupancy hint: 6 (fp32) or 4 (bf16) waves per SIMD; the bf16 histogram
// variant needs more registers (3: a tighter hint spills them to scratch).
// LDS limits the histogram variant to 6 workgroups per CU anyway.
template <int DT, bool TR>
constexpr int kStreamWaves = (DT == SS_DTYPE_F32) ? 6 : (TR ? 3 : 4);

// Static grid over (sequence, row group, chunk), for batches too small or
// too large for the balanced kernel (see use_balanced): each workgroup
// streams its chunk of every row j <= draft_len in its group, one row after
// another (one row per group for small batches). Only its histogram variant
// takes the occupancy hint: the plain one measured faster without it (B =
// 128, K = 5, every row needed: 68.0 us at 5 waves per SIMD against 71.4 at
// the 8 the hint allows), and the scalar path (rows not 16-byte aligned)
// spills under it.
template <int DT, bool VP, bool TR>
__global__ __launch_bounds__(kThreads, ((VP && TR) ? kStreamWaves<DT, TR> : 1)) void
spec_stream_kernel(Args a) {
  __shared__ f32x4 red[kWaves + 1];
  __shared__ unsigned long long hs[TR ? kHistBins : 1];
  const int tid = threadIdx.x;
  const int R = a.K + 1, nc = a.nchunks;
  const int c = blockIdx.x % nc;
  const int bg = blockIdx.x / nc;
  const int b = bg / a.ngroups, g = bg - b * a.ngroups;
  const int j0 = g * a.rows_per_wg;
  const int cstart = c * kChunk<DT>;
  // Row 0, which every valid sequence needs, is requested before the
  // sequence's parameters return.
  int d;
  float T;
  const int st = seq_check(a, b, &d, &T);  // reported by finalize
  u32x4 raw[kLoads];
  if (j0 == 0)
    load_chunk<DT, VP>(a.logits + (int64_t)b * R * a.V * Dt<DT>::kBytes, cstart,
                       a.V, tid, raw);
  int x = draft_token(a, b, j0);
  if (TR && blockIdx.x == 0 && tid == 0) *a.tcount = 0;  // rows the plan lists
  if (st) return;
  const int j1 = min(j0 + a.rows_per_wg, d + 1);
  for (int j = j0; j < j1; ++j) {
    if (j != 0)
      load_chunk<DT, VP>(a.logits + ((int64_t)b * R + j) * a.V * Dt<DT>::kBytes,
                         cstart, a.V, tid, raw);
    if (j != j0) x = draft_token(a, b, j);
    stream_row<DT, VP, TR, true>(a, b, j, d, T, c, x, raw, red, hs, NoMid{});
  }
}

constexpr int kPlanMaxB = 2048;  // sequences whose plan fits in LDS
constexpr int kPlanPer = kPlanMaxB / kThreads;

// Balanced stream: one workgroup per (sequence, chunk) of row 0, which every
// valid sequence needs, in (sequence, chunk) order. The items of rows
// 1..draft_len, (row, chunk) pairs in (sequence, row, chunk) order, are dealt
// round-robin to the same workgroups: workgroup g also takes extra items g,
// g + n0, g + 2 n0, ... (n0 = B x nchunks). The workgroups with extra work are
// therefore the first ones dispatched, and a sequence with several rows is
// spread over many workgroups instead of being streamed row after row by
// one. Every workgroup learns the number of extra rows E from the draft
// lengths (loaded while its row-0 chunk is in flight); only
// those with extra items build the exclusive prefix of draft lengths in LDS
// that maps an item to its sequence and row. (A persistent grid that deals
// every item round-robin runs its workgroups in lock-step rounds and was
// measured slower; so was handing items out with atomic counters.)
struct Item {
  int b, j, c;
};

// Item x of rows >= 1: the largest b with pre[b] <= x / nc.
__device__ __forceinline__ Item decode_extra(int x, int nc, int B, const int* pre) {
  Item t;
  const int r = x / nc;
  t.c = x - r * nc;
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    const int m = (lo + hi + 1) >> 1;
    if (pre[m] <= r) lo = m;
    else hi = m - 1;
  }
  t.b = lo;
  t.j = r - pre[lo] + 1;
  return t;
}

// Extra rows of one sequence: draft_len when it is in [1, K], else 0
// (invalid lengths are reported by finalize and need no rows).
__device__ __forceinline__ int extra_rows(const Args& a, int b) {
  const int v = a.draft_len[b] + a.dl_offset;
  return (v >= 1 && v <= a.K) ? v : 0;
}


template <int DT, bool VP, bool TR>
__global__ __launch_bounds__(kThreads, (kStreamWaves<DT, TR>)) void
spec_stream_balanced_kernel(Args a) {
  __shared__ f32x4 red[kWaves + 1];
  __shared__ unsigned long long hs[TR ? kHistBins : 1];
  __shared__ int pre[kPlanMaxB + 1];
  __shared__ int wsum[kWaves];
  const int tid = threadIdx.x, w = tid / kWave, l = tid % kWave;
  const int B = a.B, R = a.K + 1, nc = a.nchunks;
  const int n0 = B * nc;
  const int g = blockIdx.x;
  const int b0 = g / nc, c0 = g - b0 * nc;
  u32x4 raw[kLoads];
  load_chunk<DT, VP>(a.logits + (int64_t)b0 * R * a.V * Dt<DT>::kBytes,
                     c0 * kChunk<DT>, a.V, tid, raw);
  if (TR && g == 0 && tid == 0) *a.tcount = 0;  // rows the plan lists
  int d;
  float T;
  int st = seq_check(a, b0, &d, &T);  // reported by finalize
  int part = 0;
#pragma unroll
  for (int i = 0; i < kPlanPer; ++i) {
    const int b = tid + i * kThreads;
    if (b < B) part += extra_rows(a, b);
  }
  if (st == 0) stream_row<DT, VP, TR, false>(a, b0, 0, d, T, c0, -1, raw, red, hs, NoMid{});
  part = (int)wave_sum((float)part);  // exact: < 2^24
  if (l == 0) wsum[w] = part;
  __syncthreads();
  int E = 0;
  for (int i = 0; i < kWaves; ++i) E += wsum[i];
  const int nx = E * nc;  // extra items
  if (g >= nx) return;
  // Exclusive prefix of extra rows, kPlanPer consecutive sequences a thread.
  int tsum = 0;
#pragma unroll
  for (int i = 0; i < kPlanPer; ++i) {
    const int b = tid * kPlanPer + i;
    if (b < B) {
      const int v = extra_rows(a, b);
      pre[b] = v;
      tsum += v;
    }
  }
  const int incl = (int)wave_inclusive_sum((float)tsum);
  __syncthreads();  // wsum[0] has been read
  if (l == kWave - 1) wsum[w] = incl;
  __syncthreads();
  int base = incl - tsum;
  for (int i = 0; i < w; ++i) base += wsum[i];
#pragma unroll
  for (int i = 0; i < kPlanPer; ++i) {
    const int b = tid * kPlanPer + i;
    if (b < B) {
      const int v = pre[b];
      pre[b] = base;
      base += v;
    }
  }
  __syncthreads();
  for (int x = g; x < nx; x += n0) {
    const Item t = decode_extra(x, nc, B, pre);
    load_chunk<DT, VP>(a.logits + ((int64_t)t.b * R + t.j) * a.V * Dt<DT>::kBytes,
                       t.c * kChunk<DT>, a.V, tid, raw);
    st = seq_check(a, t.b, &d, &T);
    if (st == 0) stream_row<DT, VP, TR, false>(a, t.b, t.j, d, T, t.c, -1, raw, red, hs, NoMid{});
  }
}

// Workgroups the stream grid aims for: enough to keep every CU busy with
// several resident workgroups.
constexpr int64_t kTargetWorkgroups = 4096;

// Which kernel streams the rows.
//  - Fewer (sequence, chunk) pairs than kTargetWorkgroups: the row-0
//    workgroups alone do not fill the chip a few times over, and the
//    balanced kernel's extra items, taken one after another by the same
//    workgroups, would form its tail. Every (sequence, row, chunk) then gets
//    a workgroup of its own (rows past a sequence's draft length exit at
//    once). Measured at V = 151936: B = 64, K = 3 with most drafts full
//    20.2 us against 25.2; B = 32, K = 5 bf16 with few rows 7.4 against 9.8;
//    B = 128, K = 5 with every row needed 71.6 against 81.7.
//  - Up to kPlanMaxB sequences otherwise: the balanced kernel, which needs
//    no workgroup for the many rows that drafts leave unused (B = 256,
//    K = 3 with 277 of 1024 rows needed: 29.7 us against 30.5 for the full
//    grid; with no drafts 27.3 against 29.3).
//  - Draft trees: a tree's nodes usually all need their rows, so every
//    (sequence, node, chunk) gets a workgroup at any batch size (B = 256,
//    8-node trees: 198 us per verification call against 210).
//  - Larger batches: (sequence, row group, chunk), each workgroup streaming
//    its chunk of the rows of its group one after another.
inline bool tree_rows(const Args& a) { return a.dl_status == SS_ST_TREE; }

inline bool use_balanced(const Args& a) {
  return !tree_rows(a) && a.B <= kPlanMaxB &&
         (int64_t)a.B * a.nchunks >= kTargetWorkgroups;
}

inline void set_row_groups(Args& a) {
  const int R = a.K + 1;
  const int64_t base = (int64_t)a.B * a.nchunks;
  const int ngroups = (base < kTargetWorkgroups || tree_rows(a))
                          ? R
                          : (int)std::min<int64_t>(R, (kTargetWorkgroups + base - 1) / base);
  a.rows_per_wg = (R + ngroups - 1) / ngroups;
  a.ngroups = (R + a.rows_per_wg - 1) / a.rows_per_wg;
}

template <int DT, bool VP, bool TR>
int launch_stream_t(const Args& a, hipStream_t s) {
  if (use_balanced(a)) {
    hipLaunchKernelGGL((spec_stream_balanced_kernel<DT, VP, TR>),
                       dim3((unsigned)(a.B * a.nchunks)), dim3(kThreads), 0, s, a);
    return check_launch("spec_stream");
  }
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
  set_row_groups(a);
  return f32 ? (vp ? launch_stream_tr<SS_DTYPE_F32, true>(a, s)
                   : launch_stream_tr<SS_DTYPE_F32, false>(a, s))
             : (vp ? launch_stream_tr<SS_DTYPE_BF16, true>(a, s)
                   : launch_stream_tr<SS_DTYPE_BF16, false>(a, s));
}

}  // namespace specsam
