// Definitions shared by the verification kernels (stream.hip, verify.hip):
// sizes, the 16-byte load layout of a chunk, the kernel argument block and
// the per-sequence checks.
#pragma once

#include <climits>
#include <cmath>

#include "sam_device.h"

namespace specsam {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kLoads = 8;  // 16-byte loads in flight per lane
constexpr int kChunkBytes = kThreads * kLoads * 16;  // 32 KiB per workgroup
constexpr int kMaxRows = SS_MAX_K + 1;
constexpr int kMaxV = 1 << 21;
constexpr int kMaxChunks = kMaxV / (kChunkBytes / 4);  // 256 (fp32 chunks)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -INFINITY;

// Truncation (top-k / top-p) of the target distribution.
//   Window histogram: each chunk counts its finite logits, and sums their
//   probability (relative to the chunk's max, fixed point with 31 fraction
//   bits), in kHistBins bins of 1/kBinsPerOctave octave of probability,
//   starting at the bin of the chunk max (32 octaves). Bins lie on one grid
//   for all chunks of a row: the bin of logit l is floor(-l * log2e/T *
//   kBinsPerOctave) (abs_bin), so a chunk's window is a shift of the row's.
//   One bin is a 64-bit word: count in bits 48..63, mass in bits 0..47. Logits
//   below the window are not binned; the chunk's header holds its finite
//   count, and its total mass is the stream partial's sum.
//   Band: the window bins [lo, hi] whose logits a chunk copies to its
//   candidate segment (at most kSegCap of them), chosen from the chunk's own
//   histogram; hi = kRestBin takes every bin from lo down, past the window
//   too.
constexpr int kHistBins = 256;
constexpr int kBinsPerOctave = 8;
constexpr int kRestBin = kHistBins;  // "beyond the window"
constexpr int kCandCap = 8192;       // candidates per row held in LDS
constexpr int kSegCap = 1024;        // logits per (row, chunk) segment
constexpr int kBandHalf = 4;         // top-p band: bins either side of the estimate
constexpr int kNoBand = 1;           // packed band (lo = 1, hi = 0): none
constexpr float kFixScale = 2147483648.0f;  // 2^31
// A top-p band that starts within this many bins (12 octaves) of the chunk
// max takes its weight above the band from the histogram's masses: each
// token's mass is rounded to 2^-32 of the chunk max, and every token above
// the band weighs at least 2^-12 of it, so the sum is off by at most 2^-20
// of itself. Deeper bands sum the tokens' weights instead.
constexpr int kFixAboveBins = 12 * kBinsPerOctave;
constexpr unsigned long long kCountOne = 1ull << 48;
constexpr unsigned long long kMassMask = kCountOne - 1;

template <int DT>
struct Dt;
template <>
struct Dt<SS_DTYPE_F32> {
  static constexpr int kBytes = 4;
};
template <>
struct Dt<SS_DTYPE_BF16> {
  static constexpr int kBytes = 2;
};
template <int DT>
constexpr int kVec = 16 / Dt<DT>::kBytes;  // elements per 16-byte load
template <int DT>
constexpr int kChunk = kChunkBytes / Dt<DT>::kBytes;  // elements per chunk
template <int DT>
constexpr int kSeg = kChunk<DT> / kThreads;  // elements per lane in a re-read

// Element k of a 16-byte vector, widened to float (bf16 exactly).
template <int DT>
__device__ __forceinline__ float elem(const u32x4& r, int k) {
  if constexpr (DT == SS_DTYPE_F32) {
    return __uint_as_float(r[k]);
  } else {
    const unsigned w = r[k >> 1];
    return __uint_as_float((k & 1) ? (w & 0xffff0000u) : (w << 16));
  }
}

template <int DT>
__device__ __forceinline__ float load_one(const unsigned char* base, int64_t i) {
  if constexpr (DT == SS_DTYPE_F32) {
    return reinterpret_cast<const float*>(base)[i];
  } else {
    const unsigned short h = reinterpret_cast<const unsigned short*>(base)[i];
    return __uint_as_float((unsigned)h << 16);
  }
}

// Index (within the row) of element k of load `it` of lane `tid`: load it of
// lane tid covers kVec consecutive elements at cstart + (it*256 + tid)*kVec,
// so one wavefront's load is one contiguous 1 KiB request. Token order in a
// chunk is therefore (it, lane, k); each lane sees its elements in increasing
// index order, which the argmax relies on for its lowest-index tie rule and
// the draw for its scan. The scalar path (rows not 16-byte aligned) uses the
// same layout with element-wise loads.
template <int DT, bool VP>
__device__ __forceinline__ int elem_index(int cstart, int tid, int it, int k) {
  return cstart + (it * kThreads + tid) * kVec<DT> + k;
}

// load_chunk in two phases, without a branch (vector rows, VP): the loads
// (load_chunk_flat: the index of a vector past the row's end is clamped into
// the row), then, once every load of the kernel's batch is requested,
// chunk_tail_neginf replaces the vectors past the end by -inf words. The
// branches of load_chunk's tail path, a select next to its load, and the
// register copies where load_chunk's two paths join each wait for the loads
// in flight; split this way, all of them are in flight together. A vector
// is wholly in the row or wholly past its end, as V is a multiple of kVec.
template <int DT, bool NT = true>
__device__ __forceinline__ void load_chunk_flat(const unsigned char* row, int cstart,
                                                int V, int tid, u32x4 (&raw)[kLoads]) {
  const u32x4* p = reinterpret_cast<const u32x4*>(row + (int64_t)cstart * Dt<DT>::kBytes);
  const int last = (V - cstart) / kVec<DT> - 1;
#pragma unroll
  for (int it = 0; it < kLoads; ++it) {
    const int vi = min(it * kThreads + tid, last);
    raw[it] = NT ? __builtin_nontemporal_load(p + vi) : p[vi];
  }
}
template <int DT>
__device__ __forceinline__ void chunk_tail_neginf(int cstart, int V, int tid,
                                                  u32x4 (&raw)[kLoads]) {
  constexpr unsigned kNegInfWord =
      DT == SS_DTYPE_F32 ? 0xff800000u : 0xff80ff80u;
  const int rem = V - cstart;
#pragma unroll
  for (int it = 0; it < kLoads; ++it) {
    const bool in = (it * kThreads + tid) * kVec<DT> < rem;
    const u32x4 x = raw[it];
    raw[it] = u32x4{in ? x[0] : kNegInfWord, in ? x[1] : kNegInfWord,
                    in ? x[2] : kNegInfWord, in ? x[3] : kNegInfWord};
  }
}

// Loads one chunk of a row into registers. Elements past V read as -inf.
// NT: non-temporal loads for the streaming pass (measured faster there:
// with ordinary loads the c3 stream pass, B = 256, V = 151936, took 33.6 us
// against 29.4, and the finalize's re-read of one chunk per sequence gained
// nothing); the draw's single-chunk re-read uses ordinary loads, which can
// still find the chunk in the memory-side cache.
template <int DT, bool VP, bool NT = true>
__device__ __forceinline__ void load_chunk(const unsigned char* row, int cstart,
                                           int V, int tid, u32x4 (&raw)[kLoads]) {
  constexpr unsigned kNegInfWord =
      DT == SS_DTYPE_F32 ? 0xff800000u : 0xff80ff80u;
  if constexpr (VP) {
    const u32x4* p = reinterpret_cast<const u32x4*>(
        row + (int64_t)cstart * Dt<DT>::kBytes);
    const int rem = V - cstart;
    if (rem >= kChunk<DT>) {
#pragma unroll
      for (int it = 0; it < kLoads; ++it)
        raw[it] = NT ? __builtin_nontemporal_load(p + it * kThreads + tid)
                     : p[it * kThreads + tid];
    } else {
#pragma unroll
      for (int it = 0; it < kLoads; ++it) {
        const int e = (it * kThreads + tid) * kVec<DT>;
        if (e < rem)
          raw[it] = NT ? __builtin_nontemporal_load(p + it * kThreads + tid)
                       : p[it * kThreads + tid];
        else
          raw[it] = u32x4{kNegInfWord, kNegInfWord, kNegInfWord, kNegInfWord};
      }
    }
  } else {
#pragma unroll
    for (int it = 0; it < kLoads; ++it) {
      unsigned w[4] = {kNegInfWord, kNegInfWord, kNegInfWord, kNegInfWord};
#pragma unroll
      for (int k = 0; k < kVec<DT>; ++k) {
        const int i = elem_index<DT, false>(cstart, tid, it, k);
        if (i < V) {
          if constexpr (DT == SS_DTYPE_F32) {
            w[k] = __builtin_nontemporal_load(
                reinterpret_cast<const unsigned*>(row) + i);
          } else {
            const unsigned h = __builtin_nontemporal_load(
                reinterpret_cast<const unsigned short*>(row) + i);
            w[k >> 1] = (k & 1) ? ((w[k >> 1] & 0xffffu) | (h << 16))
                                : ((w[k >> 1] & 0xffff0000u) | h);
          }
        }
      }
      raw[it] = u32x4{w[0], w[1], w[2], w[3]};
    }
  }
}


struct Args {
  const unsigned char* logits;
  int B, K, V, nchunks;
  int ngroups;      // row lanes of the stream grid (set by launch_stream)
  const int32_t* draft;
  const int32_t* draft_len;
  int dl_offset;    // rows needed = draft_len[b] + dl_offset + 1 (trees: -1)
  int dl_status;    // status bit for a length outside [0, K]
  const float* q;
  const float* temperature;
  const float* uniforms;
  int32_t* out;
  int32_t* nem;
  float* p_draft;
  float* logprob;   // [B, K+1] or NULL: log-probabilities of emitted tokens
  const int32_t* top_k;  // [B] or NULL
  const float* top_p;    // [B] or NULL
  int32_t* status;
  f32x4* partials;  // [B*(K+1)*nchunks]: (max, sumexp | nan flag, l[x], argidx)
  f32x4* wparts;    // [B*(K+1)*nchunks] or NULL: an untruncated T > 0 chunk's
                    //   sums per quarter (loads 2q, 2q+1), relative to its max
  i32x4* seqinfo;   // [B]: (rejected row + 1 or 0, m, S, log2e/T)
  float* rpart;     // [B*nchunks] residual chunk sums
  f32x4* rqpart;    // [B*nchunks] residual sums per quarter of the chunk
  f32x4* seqinfo2;  // [B]: (truncation threshold, untruncated S, 0, 0)
  // Truncation workspace (NULL unless top_k or top_p is given), per row
  // (b*(K+1) + j) and per (row, chunk):
  unsigned long long* hist;  // [rows*nchunks*kHistBins] window histograms
  i32x4* hhdr;      // [rows*nchunks]: (window start bin, finite count,
                    //   band lo | hi << 16, logits in the band's segment)
  float* cand;      // [rows*nchunks*segcap] the band's logits per chunk
  int segcap;       // logits a chunk's segment holds: min(kSegCap, V)
  float* tpart;     // [rows*nchunks] the stream pass: weight above the band
                    //   (relative to the chunk max); the selection: kept
                    //   weight per chunk (relative to the row max)
  f32x4* tinfo;     // [rows]: (threshold logit, kept mass, active, 0)
  // Fused automaton step (sam == nullptr when only verifying).
  unsigned char* sam;
  int max_len;
  SamLayout sl;
  int32_t* next_draft;
  int32_t* next_draft_len;
  int32_t* next_match_len;
};

// Per-sequence checks that need device data.
__device__ __forceinline__ int seq_check(const Args& a, int b, int* d, float* T) {
  *d = a.draft_len[b] + a.dl_offset;
  *T = a.temperature[b];
  int st = 0;
  if (*d < 0 || *d > a.K) st |= a.dl_status;
  // T = 0 is greedy; otherwise T must be a finite normal positive float so
  // that log2(e)/T stays finite.
  if (!(*T == 0.0f || (*T >= 1.17549435e-38f && isfinite(*T))))
    st |= SS_ST_TEMPERATURE;
  if (*T > 0.0f && a.uniforms == nullptr) st |= SS_ST_NO_UNIFORMS;
  if (a.top_p) {
    const float p = a.top_p[b];
    if (!(p > 0.0f && p <= 1.0f)) st |= SS_ST_TOP_P;
  }
  return st;
}

// Whether sequence b's target distribution is truncated: T > 0 and top-k
// with 1 <= k < V, or top-p below 1.
__device__ __forceinline__ bool trunc_active(const Args& a, int b, float T) {
  if (!(T > 0.0f)) return false;
  const int k = a.top_k ? a.top_k[b] : 0;
  const float p = a.top_p ? a.top_p[b] : 1.0f;
  return (k >= 1 && k < a.V) || p < 1.0f;
}

// Histogram bin of a finite logit on the row's absolute grid (see kHistBins):
// floor(l * ns), ns = -log2e/T * kBinsPerOctave (bin_scale), the product
// clamped to +-1e9 before the floor. Every kernel computes it with these
// same operations, so a token's bin is the same wherever it is computed.
// Since floor(t) >= n exactly when t >= n for an integer n, and the clamp
// does not change that comparison for |n| < 1e9, a bin range [n0, n1] holds
// exactly the tokens whose product l * ns lies in [n0, n1 + 1) (so -inf,
// whose product is +inf, and NaN fall in no finite range).
__device__ __forceinline__ float bin_scale(float kk) { return -kk * (float)kBinsPerOctave; }
__device__ __forceinline__ float band_t(float l, float ns) {
  return __builtin_amdgcn_fmed3f(l * ns, -1.0e9f, 1.0e9f);
}
// floor(x) as an int, in one instruction (exact for |x| < 2^31).
__device__ __forceinline__ int floor_i32(float x) {
  int r;
  asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(r) : "v"(x));
  return r;
}
__device__ __forceinline__ int abs_bin_s(float l, float ns) { return floor_i32(band_t(l, ns)); }
__device__ __forceinline__ int abs_bin(float l, float kk) { return abs_bin_s(l, bin_scale(kk)); }

// Neighbour of f on the ordered line of floats (dir = +1: next larger, -1:
// next smaller; -0 and +0 are adjacent points).
__device__ __forceinline__ float float_step(float f, int dir) {
  unsigned u = __float_as_uint(f);
  unsigned k = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  k += (unsigned)dir;
  u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
  return __uint_as_float(u);
}

// The largest logit v whose product v * ns (rounded, as every bin test
// computes it) is at least c, for ns < 0. The rounded product does not
// increase with v, so {v : v * ns >= c} is exactly {v <= result}: a test of
// a logit against the result is the product test. Found from c / ns by
// single steps along the floats; false if it did not settle within a few
// (degenerate scales), and then the caller must not use it.
__device__ __forceinline__ bool logit_upto(float c, float ns, float* out) {
  float v = (c == INFINITY) ? (3.40282347e38f / ns) : (c / ns);
  int i = 0;
  for (; i < 8 && !(v * ns >= c); ++i) v = float_step(v, -1);
  for (; i < 16; ++i) {
    const float u = float_step(v, 1);
    if (!(u * ns >= c)) break;
    v = u;
  }
  *out = v;
  return (v * ns >= c) && !(float_step(v, 1) * ns >= c);
}

// Order-preserving key of a float (larger float, larger key; -0 as +0).
__device__ __forceinline__ unsigned fkey(float l) {
  const unsigned u = __float_as_uint(l == 0.0f ? 0.0f : l);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float fkey_inv(unsigned k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// (value, index) merge: larger value wins, the lower index on equal values.
__device__ __forceinline__ void argmax_merge(float& v, int& i, float ov, int oi) {
  if (ov > v || (ov == v && oi < i)) {
    v = ov;
    i = oi;
  }
}

// Online-softmax merge of (max, sum exp2((x-max)*kk)) pairs.
__device__ __forceinline__ void lse_merge(float& m, float& s, float om, float os,
                                          float kk) {
  const float M = fmaxf(m, om);
  const float Mb = (M == kNegInf) ? 0.0f : M;
  s = s * fast_exp2((m - Mb) * kk) + os * fast_exp2((om - Mb) * kk);
  m = M;
}

// Wavefront reductions of (value, index) by argmax_merge and of (max, sum)
// by lse_merge; every lane ends with the result.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  float fi = __int_as_float(i);
  wave_reduce2(v, fi, kNegInf, __int_as_float(INT_MAX),
               [](float& x, float& y, float ox, float oy) {
                 int iy = __float_as_int(y);
                 argmax_merge(x, iy, ox, __float_as_int(oy));
                 y = __int_as_float(iy);
               });
  i = __float_as_int(fi);
}

__device__ __forceinline__ void wave_lse(float& m, float& s, float kk) {
  wave_reduce2(m, s, kNegInf, 0.0f, [kk](float& x, float& y, float ox, float oy) {
    lse_merge(x, y, ox, oy, kk);
  });
}

// Partials and residual sums are written by one kernel and read by the next
// one on the same stream; plain accesses suffice.
__device__ __forceinline__ f32x4 load_partial(const f32x4* p) { return *p; }
__device__ __forceinline__ float load_f32(const float* p) { return *p; }

// Launches the stream pass (stream.hip): one partial per (row, chunk) of the
// rows each sequence needs. f32 selects fp32 logits (else bf16); vp the
// 16-byte vector path (rows 16-byte aligned and V a multiple of the vector).
int launch_stream(Args a, bool f32, bool vp, hipStream_t s);

// Launches the tree finalize kernel (tree.hip) after the stream pass over
// every node's row: one workgroup per sequence.
int launch_tree_finalize(const Args& a, bool f32, bool vp, const int32_t* tokens,
                         const int32_t* parent, int32_t* out_nodes, hipStream_t s);

// Launches the truncation selection (trunc.hip) after the stream pass: the
// threshold and the kept weight per chunk of every truncated row.
int launch_truncation(const Args& a, bool f32, bool vp, hipStream_t s);

}  // namespace specsam
