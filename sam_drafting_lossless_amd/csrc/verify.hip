// Batched lossless verification of K drafted tokens against target logits.
//
// Method ([P2] m.nxbn.cn guide §2.2; [P3] gogongxt notes "贪婪采样",
// "拒绝采样", "SGLang 的实现"; [P1] cann-recipes-train article §1.1 and
// §3.1.2): the target scores K+1 positions in one forward. Drafts are judged
// in order; T = 0 accepts a draft iff it is the target argmax, T > 0 accepts
// x_j iff u_j <= p_j(x_j) / q_j(x_j). The first rejection emits a token from
// max(0, p - q) normalised (p with x_j removed for one-hot drafts); if every
// draft passes, a bonus token comes from the last row.
//
// Design for gfx950 (the hot path is one HBM stream over B*(K+1)*V logits):
//   pass 1  grid over (row, chunk); each 256-thread workgroup streams one
//           32 KiB chunk with non-temporal 16-byte loads (8 in flight per
//           lane) and writes one partial: (max, argmax) at T = 0, or (max,
//           sum exp2((l-max)*log2e/T)) at T > 0. Rows j > draft_len are
//           skipped. The last workgroup of a sequence to finish (device-scope
//           counter with release/acquire fences) combines the partials, runs
//           the accept scan as a wavefront ballot, writes the outputs and,
//           for one-hot drafts or the bonus, draws the token: it picks the
//           chunk from the rescaled partials and re-reads only that chunk.
//   pass 2  only when q is given: a grid over (sequence, chunk) of the
//           rejected row computes chunk sums of max(0, p - q); the last
//           workgroup picks the chunk and re-reads it for the draw.
#include <climits>
#include <cmath>

#include "internal.h"

namespace specsam {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kLoads = 8;  // 16-byte loads in flight per lane
constexpr int kChunkBytes = kThreads * kLoads * 16;  // 32 KiB per workgroup
constexpr int kMaxRows = SS_MAX_K + 1;
constexpr int kMaxV = 1 << 21;
constexpr int kMaxChunks = kMaxV / (kChunkBytes / 4);  // 256 (fp32 chunks)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -INFINITY;

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

// Index (within the row) of element k of load `it` of lane `tid`. Each lane
// sees its elements in increasing index order (it, then k), which the argmax
// relies on for its lowest-index tie rule.
//   VP (vector path): load it of lane tid covers kVec consecutive elements at
//                     cstart + (it*256 + tid)*kVec: one coalesced 4 KiB wave
//                     request per load.
//   scalar path:      element e = it*kVec + k sits at cstart + e*256 + tid.
template <int DT, bool VP>
__device__ __forceinline__ int elem_index(int cstart, int tid, int it, int k) {
  if constexpr (VP)
    return cstart + (it * kThreads + tid) * kVec<DT> + k;
  else
    return cstart + (it * kVec<DT> + k) * kThreads + tid;
}

// Loads one chunk of a row into registers. Elements past V read as -inf.
template <int DT, bool VP>
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
        raw[it] = __builtin_nontemporal_load(p + it * kThreads + tid);
    } else {
#pragma unroll
      for (int it = 0; it < kLoads; ++it) {
        const int e = (it * kThreads + tid) * kVec<DT>;
        if (e < rem)
          raw[it] = __builtin_nontemporal_load(p + it * kThreads + tid);
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
  const int32_t* draft;
  const int32_t* draft_len;
  const float* q;
  const float* temperature;
  const float* uniforms;
  int32_t* out;
  int32_t* nem;
  float* p_draft;
  int32_t* status;
  f32x4* partials;  // [B*(K+1)*nchunks]: (max, sumexp | nan flag, argval, argidx)
  i32x4* seqinfo;   // [B]: (rejected row + 1 or 0, m, S, log2e/T) for pass 2
  unsigned* ctr1;   // [B] pass-1 completion counters (zero between calls)
  unsigned* ctr2;   // [B] pass-2 completion counters
  float* rpart;     // [B*nchunks] residual chunk sums
};

// Host-invisible per-sequence checks, identical in every workgroup.
__device__ __forceinline__ int seq_check(const Args& a, int b, int* d, float* T) {
  *d = a.draft_len[b];
  *T = a.temperature[b];
  int st = 0;
  if (*d < 0 || *d > a.K) st |= SS_ST_DRAFT_LEN;
  // T = 0 is greedy; otherwise T must be a finite normal positive float so
  // that log2(e)/T stays finite.
  if (!(*T == 0.0f || (*T >= 1.17549435e-38f && *T <= 3.4e38f)))
    st |= SS_ST_TEMPERATURE;
  if (*T > 0.0f && a.uniforms == nullptr) st |= SS_ST_NO_UNIFORMS;
  return st;
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

// ---------------------------------------------------------------------------
// Draw from a row given chunk weights. Shared by the one-hot / bonus draw
// (weights exp2((l-m)*kk), optionally with one token removed) and the
// residual draw (weights max(0, exp2((l-m)*kk)/S - q)).
//
// Step 1 (wave 0): inclusive scan of the chunk weights in chunk order, pick
// the first chunk whose running sum exceeds u*total (strict), or the last
// chunk with positive weight if rounding leaves none. Step 2 (all lanes):
// re-read that chunk as 256 contiguous segments, scan the lane sums, and let
// the lane whose interval holds the target find the first token whose running
// sum exceeds it. Ties in rounding fall back to the last positive weight.
// ---------------------------------------------------------------------------
struct DrawShared {
  float W[kMaxChunks];
  float cum[kMaxChunks];
  float wsum[kWaves];
  int wlast[kWaves];
  float t_in;
  int chunk;
  int result;
};

template <int DT, bool RESIDUAL>
__device__ int draw_row(const Args& a, DrawShared& sh, int b, int r, int excl,
                        float m, float S, float kk, float u, int nc) {
  const int tid = threadIdx.x, w = tid / kWave, l = tid % kWave;
  const int R = a.K + 1;
  const unsigned char* row =
      a.logits + ((int64_t)(b * R + r) * a.V) * Dt<DT>::kBytes;
  const float* qrow = RESIDUAL ? a.q + (int64_t)(b * a.K + r) * a.V : nullptr;
  const float invS = RESIDUAL ? 1.0f / S : 0.0f;
  if (w == 0) {
    float wx = 0.0f;
    int cx = -1;
    if (!RESIDUAL && excl >= 0) {
      wx = fast_exp2((load_one<DT>(row, excl) - m) * kk);
      cx = excl / kChunk<DT>;
    }
    float carry = 0.0f;
    for (int g = 0; g < nc; g += kWave) {
      const int c = g + l;
      float W = 0.0f;
      if (c < nc) {
        if constexpr (RESIDUAL) {
          W = a.rpart[(int64_t)b * nc + c];
        } else {
          const f32x4 P = a.partials[(int64_t)(b * R + r) * nc + c];
          W = P.y * fast_exp2((P.x - m) * kk);
          if (c == cx) W = fmaxf(0.0f, W - wx);
        }
      }
      const float inc = wave_inclusive_sum(W) + carry;
      if (c < nc) {
        sh.W[c] = W;
        sh.cum[c] = inc;
      }
      carry = __shfl(inc, kWave - 1, kWave);
    }
    const float t = u * carry;
    int chosen = -1, lastpos = -1;
    for (int g = 0; g < nc && chosen < 0; g += kWave) {
      const int c = g + l;
      const bool ok = c < nc;
      const unsigned long long hit = __ballot(ok && sh.cum[c] > t);
      const unsigned long long pos = __ballot(ok && sh.W[c] > 0.0f);
      if (hit) chosen = g + __ffsll((long long)hit) - 1;
      if (pos) lastpos = g + 63 - __clzll((long long)pos);
    }
    if (l == 0) {
      if (chosen >= 0) {
        sh.chunk = chosen;
        sh.t_in = t - (sh.cum[chosen] - sh.W[chosen]);
      } else {
        sh.chunk = lastpos;  // rounding: take the last positive weight
        sh.t_in = INFINITY;
      }
    }
  }
  __syncthreads();
  const int c = sh.chunk;
  if (c < 0) return -1;  // no positive weight at all (caller guards)
  const float t_in = sh.t_in;
  // Contiguous segment of this lane within the chunk.
  const int s0 = c * kChunk<DT> + tid * kSeg<DT>;
  const int s1 = min(s0 + kSeg<DT>, a.V);
  float tsum = 0.0f;
  int tlast = -1;
  for (int i = s0; i < s1; ++i) {
    float wi;
    if constexpr (RESIDUAL)
      wi = fmaxf(0.0f, fast_exp2((load_one<DT>(row, i) - m) * kk) * invS - qrow[i]);
    else
      wi = (i == excl) ? 0.0f : fast_exp2((load_one<DT>(row, i) - m) * kk);
    tsum += wi;
    if (wi > 0.0f) tlast = i;
  }
  // Block-wide inclusive scan of lane sums.
  float inc = wave_inclusive_sum(tsum);
  if (l == kWave - 1) sh.wsum[w] = inc;
  int wl = tlast;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) wl = max(wl, __shfl_xor(wl, o, kWave));
  if (l == 0) sh.wlast[w] = wl;
  __syncthreads();
  float wbase = 0.0f;
  for (int i = 0; i < w; ++i) wbase += sh.wsum[i];
  inc += wbase;
  float exc = __shfl_up(inc, 1, kWave);
  if (l == 0) exc = wbase;
  if (tid == 0) {
    int cl = -1;
    for (int i = 0; i < kWaves; ++i) cl = max(cl, sh.wlast[i]);
    sh.result = cl;  // default: last positive weight of the chunk
  }
  __syncthreads();
  if (exc <= t_in && t_in < inc) {
    const float tl = t_in - exc;
    float run = 0.0f;
    int found = tlast;
    for (int i = s0; i < s1; ++i) {
      float wi;
      if constexpr (RESIDUAL)
        wi = fmaxf(0.0f,
                   fast_exp2((load_one<DT>(row, i) - m) * kk) * invS - qrow[i]);
      else
        wi = (i == excl) ? 0.0f : fast_exp2((load_one<DT>(row, i) - m) * kk);
      run += wi;
      if (run > tl) {
        found = i;
        break;
      }
    }
    sh.result = found;  // at most one lane's interval holds t_in
  }
  __syncthreads();
  return sh.result;
}

// ---------------------------------------------------------------------------
// Last workgroup of sequence b: combine partials, decide, emit.
// ---------------------------------------------------------------------------
struct FinalShared {
  float m[kMaxRows];
  float s[kMaxRows];
  int idx[kMaxRows];
  int bad[kMaxRows];
  int acc_len;
  int st;
  DrawShared draw;
};

template <int DT>
__device__ void finalize(const Args& a, FinalShared& sh, int b, int d, float T,
                         float kk) {
  const int tid = threadIdx.x, w = tid / kWave, l = tid % kWave;
  const int R = a.K + 1, nc = a.nchunks;
  const bool greedy = (T == 0.0f);
  for (int j = w; j <= d; j += kWaves) {
    const f32x4* P = a.partials + (int64_t)(b * R + j) * nc;
    if (greedy) {
      float bv = kNegInf;
      int bi = INT_MAX, nan = 0;
      for (int c = l; c < nc; c += kWave) {
        const f32x4 p = P[c];
        argmax_merge(bv, bi, p.x, __float_as_int(p.w));
        nan |= (p.y != 0.0f);
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1)
        argmax_merge(bv, bi, __shfl_xor(bv, o, kWave), __shfl_xor(bi, o, kWave));
      nan = wave_or(nan);
      if (l == 0) {
        sh.m[j] = bv;
        sh.idx[j] = bi;
        sh.bad[j] = nan || bv == INFINITY || bv == kNegInf;
      }
    } else {
      float m = kNegInf, s = 0.0f;
      for (int c = l; c < nc; c += kWave) {
        const f32x4 p = P[c];
        lse_merge(m, s, p.x, p.y, kk);
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1)
        lse_merge(m, s, __shfl_xor(m, o, kWave), __shfl_xor(s, o, kWave), kk);
      if (l == 0) {
        sh.m[j] = m;
        sh.s[j] = s;
        sh.bad[j] = !(s > 0.0f) || !isfinite(s) || !isfinite(m);
      }
    }
  }
  __syncthreads();
  if (w == 0) {
    int st = 0, x = -1;
    if (l < d) {
      x = a.draft[(int64_t)b * a.K + l];
      if (x < 0 || x >= a.V) st |= SS_ST_TOKEN_RANGE;
    }
    if (l <= d && sh.bad[l]) st |= SS_ST_NONFINITE;
    st = wave_or(st);
    if (st) {
      if (l == 0) {
        atomicOr(&a.status[b], st);
        sh.st = st;
      }
    } else {
      bool acc = true;
      float px = -1.0f;
      if (l < d) {
        if (greedy) {
          acc = (x == sh.idx[l]);
        } else {
          const unsigned char* row =
              a.logits + ((int64_t)(b * R + l) * a.V) * Dt<DT>::kBytes;
          px = fast_exp2((load_one<DT>(row, x) - sh.m[l]) * kk) / sh.s[l];
          const float qx = a.q ? a.q[((int64_t)b * a.K + l) * a.V + x] : 1.0f;
          const float u = a.uniforms[(int64_t)b * R + l];
          acc = (qx > 0.0f) ? (u <= px / qx) : (px > 0.0f);
        }
      }
      // Wavefront scan of the accept flags: the first rejection ends the run.
      const unsigned long long rej = __ballot(!acc);
      const int al = rej ? __ffsll((long long)rej) - 1 : d;
      if (l < R) {
        if (l < al)
          a.out[(int64_t)b * R + l] = x;
        else if (l == al && greedy)
          a.out[(int64_t)b * R + l] = sh.idx[l];
        else if (l > al)
          a.out[(int64_t)b * R + l] = -1;
      }
      if (a.p_draft && l < a.K)
        a.p_draft[(int64_t)b * a.K + l] = (!greedy && l < d && l <= al) ? px : -1.0f;
      if (l == 0) {
        a.nem[b] = al + 1;
        sh.acc_len = al;
        sh.st = 0;
      }
    }
  }
  __syncthreads();
  if (sh.st == 0 && !greedy) {
    const int al = sh.acc_len;
    if (al < d && a.q != nullptr) {
      // Residual max(0, p - q) needs p over the whole row: pass 2 draws it.
      if (tid == 0)
        a.seqinfo[b] = i32x4{al + 1, __float_as_int(sh.m[al]),
                             __float_as_int(sh.s[al]), __float_as_int(kk)};
    } else {
      const int excl = (al < d) ? a.draft[(int64_t)b * a.K + al] : -1;
      const float u = a.uniforms[(int64_t)b * R + a.K];
      const int tok = draw_row<DT, false>(a, sh.draw, b, al, excl, sh.m[al],
                                          sh.s[al], kk, u, nc);
      if (tid == 0) a.out[(int64_t)b * R + al] = tok;
    }
  }
  if (tid == 0) a.ctr1[b] = 0u;  // leave the counter zero for the next call
}

template <int DT, bool VP>
__global__ __launch_bounds__(kThreads) void verify_pass1(Args a) {
  __shared__ f32x4 red[kWaves];
  __shared__ int last_flag;
  __shared__ FinalShared fsh;
  const int tid = threadIdx.x, w = tid / kWave, l = tid % kWave;
  const int R = a.K + 1;
  const int row = blockIdx.x / a.nchunks;
  const int c = blockIdx.x - row * a.nchunks;
  const int b = row / R, j = row - b * R;
  int d;
  float T;
  const int st = seq_check(a, b, &d, &T);
  if (st) {
    if (j == 0 && c == 0 && tid == 0) atomicOr(&a.status[b], st);
    return;
  }
  if (j > d) return;
  const bool greedy = (T == 0.0f);
  const float kk = greedy ? 0.0f : kLog2e / T;
  const int cstart = c * kChunk<DT>;
  const unsigned char* rowp = a.logits + ((int64_t)row * a.V) * Dt<DT>::kBytes;
  u32x4 raw[kLoads];
  load_chunk<DT, VP>(rowp, cstart, a.V, tid, raw);

  if (greedy) {
    float bv = kNegInf;
    int bi = INT_MAX, nan = 0;
#pragma unroll
    for (int it = 0; it < kLoads; ++it)
#pragma unroll
      for (int k = 0; k < kVec<DT>; ++k) {
        const float v = elem<DT>(raw[it], k);
        if (v > bv) {
          bv = v;
          bi = elem_index<DT, VP>(cstart, tid, it, k);
        }
        nan |= (v != v);
      }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
      argmax_merge(bv, bi, __shfl_xor(bv, o, kWave), __shfl_xor(bi, o, kWave));
    nan = wave_or(nan);
    if (l == 0) red[w] = f32x4{bv, nan ? 1.0f : 0.0f, 0.0f, __int_as_float(bi)};
    __syncthreads();
    if (tid == 0) {
      f32x4 p = red[0];
      float pv = p.x;
      int pi = __float_as_int(p.w);
      float pn = p.y;
      for (int i = 1; i < kWaves; ++i) {
        argmax_merge(pv, pi, red[i].x, __float_as_int(red[i].w));
        pn = fmaxf(pn, red[i].y);
      }
      red[0] = f32x4{pv, pn, 0.0f, __int_as_float(pi)};
    }
  } else {
    float mx = kNegInf;
#pragma unroll
    for (int it = 0; it < kLoads; ++it)
#pragma unroll
      for (int k = 0; k < kVec<DT>; ++k) mx = fmaxf(mx, elem<DT>(raw[it], k));
    const float base = (mx == kNegInf) ? 0.0f : mx;
    float s = 0.0f;
#pragma unroll
    for (int it = 0; it < kLoads; ++it)
#pragma unroll
      for (int k = 0; k < kVec<DT>; ++k)
        s += fast_exp2((elem<DT>(raw[it], k) - base) * kk);
#pragma unroll
    for (int o = 32; o > 0; o >>= 1)
      lse_merge(mx, s, __shfl_xor(mx, o, kWave), __shfl_xor(s, o, kWave), kk);
    if (l == 0) red[w] = f32x4{mx, s, 0.0f, 0.0f};
    __syncthreads();
    if (tid == 0) {
      float pm = red[0].x, ps = red[0].y;
      for (int i = 1; i < kWaves; ++i) lse_merge(pm, ps, red[i].x, red[i].y, kk);
      red[0] = f32x4{pm, ps, 0.0f, 0.0f};
    }
  }
  if (tid == 0) {
    a.partials[(int64_t)row * a.nchunks + c] = red[0];
    __threadfence();  // release the partial before counting it
    const unsigned old = atomicAdd(&a.ctr1[b], 1u);
    last_flag = (old == (unsigned)((d + 1) * a.nchunks - 1));
  }
  __syncthreads();
  if (!last_flag) return;
  __threadfence();  // acquire: every partial of this sequence is visible
  finalize<DT>(a, fsh, b, d, T, kk);
}

template <int DT, bool VP>
__global__ __launch_bounds__(kThreads) void verify_residual(Args a) {
  __shared__ float red[kWaves];
  __shared__ int last_flag;
  __shared__ DrawShared dsh;
  const int tid = threadIdx.x, w = tid / kWave, l = tid % kWave;
  const int nc = a.nchunks;
  const int b = blockIdx.x / nc;
  const int c = blockIdx.x - b * nc;
  const i32x4 info = a.seqinfo[b];
  if (info.x == 0) return;
  const int r = info.x - 1;
  const float m = __int_as_float(info.y), S = __int_as_float(info.z);
  const float kk = __int_as_float(info.w);
  const float invS = 1.0f / S;
  const int R = a.K + 1;
  const int cstart = c * kChunk<DT>;
  const unsigned char* rowp =
      a.logits + ((int64_t)(b * R + r) * a.V) * Dt<DT>::kBytes;
  const float* qrow = a.q + (int64_t)(b * a.K + r) * a.V;
  u32x4 raw[kLoads];
  load_chunk<DT, VP>(rowp, cstart, a.V, tid, raw);
  float s = 0.0f;
#pragma unroll
  for (int it = 0; it < kLoads; ++it) {
#pragma unroll
    for (int k = 0; k < kVec<DT>; ++k) {
      const int i = elem_index<DT, VP>(cstart, tid, it, k);
      if (i < a.V) {
        const float qi = __builtin_nontemporal_load(qrow + i);
        s += fmaxf(0.0f, fast_exp2((elem<DT>(raw[it], k) - m) * kk) * invS - qi);
      }
    }
  }
  s = wave_sum(s);
  if (l == 0) red[w] = s;
  __syncthreads();
  if (tid == 0) {
    float t = 0.0f;
    for (int i = 0; i < kWaves; ++i) t += red[i];
    a.rpart[(int64_t)b * nc + c] = t;
    __threadfence();
    const unsigned old = atomicAdd(&a.ctr2[b], 1u);
    last_flag = (old == (unsigned)(nc - 1));
  }
  __syncthreads();
  if (!last_flag) return;
  __threadfence();
  if (w == 0) {
    float tot = 0.0f;
    for (int cc = l; cc < nc; cc += kWave) tot += a.rpart[(int64_t)b * nc + cc];
    tot = wave_sum(tot);
    if (l == 0) red[0] = tot;
  }
  __syncthreads();
  const float total = red[0];
  const float u = a.uniforms[(int64_t)b * R + a.K];
  int tok;
  if (total > 0.0f) {
    tok = draw_row<DT, true>(a, dsh, b, r, -1, m, S, kk, u, nc);
  } else {
    // max(0, p - q) vanished everywhere (p == q): draw from p itself.
    tok = draw_row<DT, false>(a, dsh, b, r, -1, m, S, kk, u, nc);
  }
  if (tid == 0) {
    a.out[(int64_t)b * R + r] = tok;
    a.seqinfo[b] = i32x4{0, 0, 0, 0};
    a.ctr2[b] = 0u;
  }
}

// ---------------------------------------------------------------------------
// Workspace layout (bytes, each region 256-byte aligned).
// ---------------------------------------------------------------------------
struct WsLayout {
  size_t partials, seqinfo, ctr1, ctr2, rpart, total;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline int nchunks_for(int V, int dtype) {
  const int ch = dtype == SS_DTYPE_F32 ? kChunk<SS_DTYPE_F32> : kChunk<SS_DTYPE_BF16>;
  return (V + ch - 1) / ch;
}

WsLayout ws_layout(int B, int K, int V) {
  const size_t nc = (size_t)nchunks_for(V, SS_DTYPE_F32);  // the larger count
  WsLayout L;
  size_t o = 0;
  L.partials = o;
  o = align256(o + (size_t)B * (K + 1) * nc * sizeof(f32x4));
  L.seqinfo = o;
  o = align256(o + (size_t)B * sizeof(i32x4));
  L.ctr1 = o;
  o = align256(o + (size_t)B * sizeof(unsigned));
  L.ctr2 = o;
  o = align256(o + (size_t)B * sizeof(unsigned));
  L.rpart = o;
  o = align256(o + (size_t)B * nc * sizeof(float));
  L.total = o;
  return L;
}

__global__ void fill_zero_u32x4(u32x4* p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = u32x4{0u, 0u, 0u, 0u};
}

template <int DT, bool VP>
int launch(const Args& a, hipStream_t s) {
  const int64_t grid1 = (int64_t)a.B * (a.K + 1) * a.nchunks;
  if (grid1 > INT_MAX) return set_error(SS_EINVAL, "spec_verify: grid too large");
  hipLaunchKernelGGL((verify_pass1<DT, VP>), dim3((unsigned)grid1), dim3(kThreads),
                     0, s, a);
  int rc = check_launch("spec_verify pass 1");
  if (rc != SS_OK || a.q == nullptr) return rc;
  const int64_t grid2 = (int64_t)a.B * a.nchunks;
  hipLaunchKernelGGL((verify_residual<DT, VP>), dim3((unsigned)grid2),
                     dim3(kThreads), 0, s, a);
  return check_launch("spec_verify residual pass");
}

}  // namespace
}  // namespace specsam

using namespace specsam;

extern "C" size_t ss_verify_workspace_bytes(int B, int K, int V) {
  if (B < 1 || K < 1 || K > SS_MAX_K || V < 1 || V > kMaxV) return 0;
  return ws_layout(B, K, V).total;
}

extern "C" int ss_verify_workspace_init(void* workspace, size_t ws_bytes,
                                        void* stream) {
  if (!workspace || ((uintptr_t)workspace & 15))
    return set_error(SS_EINVAL, "ss_verify_workspace_init: workspace must be "
                                "non-null and 16-byte aligned");
  const size_t n = ws_bytes / 16;
  if (n == 0) return SS_OK;
  const unsigned grid = (unsigned)std::min<size_t>((n + 255) / 256, 4096);
  hipLaunchKernelGGL(fill_zero_u32x4, dim3(grid), dim3(256), 0, as_stream(stream),
                     reinterpret_cast<u32x4*>(workspace), n);
  return check_launch("ss_verify_workspace_init");
}

extern "C" int spec_verify(const void* logits, int dtype, int B, int K, int V,
                           const int32_t* draft, const int32_t* draft_len,
                           const float* q, const float* temperature,
                           const float* uniforms, int32_t* out_tokens,
                           int32_t* num_emitted, float* p_draft, int32_t* status,
                           void* workspace, size_t ws_bytes, void* stream) {
  if (B < 1 || K < 1 || K > SS_MAX_K || V < 1 || V > kMaxV)
    return set_error(SS_EINVAL,
                     "spec_verify: need B >= 1, 1 <= K <= %d, 1 <= V <= %d "
                     "(got B=%d K=%d V=%d)",
                     SS_MAX_K, kMaxV, B, K, V);
  if (dtype != SS_DTYPE_F32 && dtype != SS_DTYPE_BF16)
    return set_error(SS_EINVAL, "spec_verify: unknown dtype %d", dtype);
  if (!logits || !draft || !draft_len || !temperature || !out_tokens ||
      !num_emitted || !status || !workspace)
    return set_error(SS_EINVAL, "spec_verify: a required pointer is NULL");
  if ((uintptr_t)workspace & 15)
    return set_error(SS_EINVAL, "spec_verify: workspace must be 16-byte aligned");
  const WsLayout L = ws_layout(B, K, V);
  if (ws_bytes < L.total)
    return set_error(SS_EWORKSPACE, "spec_verify: workspace %zu < %zu bytes",
                     ws_bytes, L.total);
  unsigned char* ws = reinterpret_cast<unsigned char*>(workspace);
  Args a;
  a.logits = reinterpret_cast<const unsigned char*>(logits);
  a.B = B;
  a.K = K;
  a.V = V;
  a.nchunks = nchunks_for(V, dtype);
  a.draft = draft;
  a.draft_len = draft_len;
  a.q = q;
  a.temperature = temperature;
  a.uniforms = uniforms;
  a.out = out_tokens;
  a.nem = num_emitted;
  a.p_draft = p_draft;
  a.status = status;
  a.partials = reinterpret_cast<f32x4*>(ws + L.partials);
  a.seqinfo = reinterpret_cast<i32x4*>(ws + L.seqinfo);
  a.ctr1 = reinterpret_cast<unsigned*>(ws + L.ctr1);
  a.ctr2 = reinterpret_cast<unsigned*>(ws + L.ctr2);
  a.rpart = reinterpret_cast<float*>(ws + L.rpart);
  const int vec = dtype == SS_DTYPE_F32 ? 4 : 8;
  const bool vp = (V % vec == 0) && (((uintptr_t)logits & 15) == 0) &&
                  (q == nullptr || ((uintptr_t)q & 15) == 0);
  hipStream_t s = as_stream(stream);
  if (dtype == SS_DTYPE_F32)
    return vp ? launch<SS_DTYPE_F32, true>(a, s) : launch<SS_DTYPE_F32, false>(a, s);
  return vp ? launch<SS_DTYPE_BF16, true>(a, s) : launch<SS_DTYPE_BF16, false>(a, s);
}
