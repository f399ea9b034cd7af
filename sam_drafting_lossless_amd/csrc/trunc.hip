// Truncation of the target distribution before verification: top-k, then
// top-p on what top-k kept, then renormalisation ([P3] gogongxt notes
// "SGLang 的实现": the target probabilities pass through a top-k and a top-p
// renormalisation, with one value of each per request, before the
// speculative-sampling kernel). Read as: top-k keeps every token whose logit
// is at least the k-th largest (tied tokens kept); top-p keeps whole groups of
// equal logits from the top until the kept share of what top-k kept reaches
// top_p. A row's truncation is then one threshold logit: keep l >= threshold.
//
// Design for gfx950. Finding the k-th largest logit, or the logit where the
// running probability crosses top_p, is a selection over V values per row.
// Sorting a 152k-entry row, or a radix select that re-reads it once per
// digit, would cost several passes over HBM. Here the row is read twice:
//   stream  (stream.hip, truncated rows only) counts each chunk's logits, and
//           sums their probability, in a 256-bin window histogram on a grid
//           shared by all chunks of the row (1/8 octave of probability per
//           bin, 32 octaves below the chunk max);
//   plan    (one workgroup per row) merges the row's chunk histograms, scans
//           them from the top and picks the bin range that must hold the
//           threshold (with a margin for the histogram's rounding);
//   extract (one workgroup per row chunk) re-reads the chunk, sums the exact
//           probability of its tokens above the range and writes the tokens
//           inside the range to the chunk's own segment of the row's
//           candidate list (no atomics);
//   select  (one workgroup per row) finds the exact threshold among the
//           candidates by radix selection on order-preserving keys (8-bit
//           digits, LDS histograms of counts for top-k and of probability
//           for top-p), then adds the kept candidates' probability to their
//           chunks' sums.
// The finalize kernel then judges and draws with the per-chunk kept sums and
// the threshold. Selection first finds the bits all candidate keys share and
// radix-walks only the bits below them, so that no round piles every
// candidate into one LDS bucket. A row with more than kCandCap candidates,
// or a chunk with more than kSegCap (logits crowded into a few bins), is
// selected by scanning the row itself in each round: exact, but slower.
#include <algorithm>

#include "verify_common.h"

namespace specsam {
namespace {

constexpr float kPlanMargin = 1e-4f;  // relative slack for histogram rounding
constexpr int kKeepAll = INT_MAX;     // range start when nothing is dropped
constexpr int64_t kExtractGrid = 4096;  // extract workgroups (grid-stride)

__device__ __forceinline__ float block_sum(float v, float* scratch) {
  const int tid = threadIdx.x, w = tid / kWave, l = tid % kWave;
  v = wave_sum(v);
  __syncthreads();
  if (l == 0) scratch[w] = v;
  __syncthreads();
  float t = 0.0f;
  for (int i = 0; i < kWaves; ++i) t += scratch[i];
  return t;
}

// Row-level activity of truncation; the same test in every kernel.
struct RowCtx {
  int b, j, d;
  float T, kk;
  bool active;
};

__device__ __forceinline__ RowCtx row_ctx(const Args& a, int64_t row) {
  RowCtx r;
  const int R = a.K + 1;
  r.b = (int)(row / R);
  r.j = (int)(row - (int64_t)r.b * R);
  const int st = seq_check(a, r.b, &r.d, &r.T);
  r.active = st == 0 && r.j <= r.d && trunc_active(a, r.b, r.T);
  r.kk = r.active ? kLog2e / r.T : 0.0f;
  return r;
}

// ---------------------------------------------------------------------------
// plan: one workgroup per row; thread r owns bin r of the row window.
// ---------------------------------------------------------------------------
constexpr int kPlanBatch = 24;  // chunk histograms requested at once

__global__ __launch_bounds__(kThreads) void trunc_plan_kernel(Args a) {
  __shared__ int s_a[kMaxChunks];
  __shared__ float s_pm[kMaxChunks];
  __shared__ float scratch[2][kWaves];
  __shared__ float wtot[2][kWaves];
  __shared__ int first[3];
  __shared__ float zval[2];
  __shared__ int cabove;
  const int tid = threadIdx.x, w = tid / kWave, l = tid % kWave;
  const int64_t row = blockIdx.x;
  const int nc = a.nchunks;
  const int64_t h0 = row * nc;
  // The chunk headers and partials are requested together with the row's
  // parameters (they are in bounds for every row; an inactive row's are
  // never used).
  i32x4 hh = i32x4{0, 0, 0, 0};
  f32x4 pv = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if (tid < nc) {
    hh = a.hhdr[h0 + tid];
    pv = a.partials[h0 + tid];
  }
  const RowCtx rc = row_ctx(a, row);
  if (!rc.active) return;
  if (tid < nc) {
    s_a[tid] = hh.x;
    s_pm[tid] = pv.x;
  }
  for (int c = tid + kThreads; c < nc; c += kThreads) {
    s_a[c] = a.hhdr[h0 + c].x;
    s_pm[c] = a.partials[h0 + c].x;
  }
  if (tid < 3) first[tid] = kRestBin;
  if (tid == 0) cabove = 0;
  __syncthreads();
  float m = kNegInf;
  for (int c = 0; c < nc; ++c) m = fmaxf(m, s_pm[c]);
  const int a0 = abs_bin(m, rc.kk);
  // Totals: the finite count N from the chunk headers and the mass Z
  // (relative to the row max) from the partials.
  float tcnt = 0.0f, tmass = 0.0f;
  if (tid < nc) {
    tcnt = (float)hh.y;
    tmass = pv.y * fast_exp2((pv.x - m) * rc.kk);
  }
  for (int c = tid + kThreads; c < nc; c += kThreads) {
    const f32x4 p = a.partials[h0 + c];
    tcnt += (float)a.hhdr[h0 + c].y;
    tmass += p.y * fast_exp2((p.x - m) * rc.kk);
  }
  // Merge: bin r of the row is bin r - (a_c - a0) of chunk c. The words of
  // kPlanBatch chunks are requested together.
  float cnt = 0.0f, mass = 0.0f;
  for (int c0 = 0; c0 < nc; c0 += kPlanBatch) {
    unsigned long long wb[kPlanBatch];
#pragma unroll
    for (int u = 0; u < kPlanBatch; ++u) {
      const int c = c0 + u;
      wb[u] = 0;
      if (c < nc) {
        const int jb = tid - (s_a[c] - a0);
        if (jb >= 0 && jb < kHistBins) wb[u] = a.hist[(h0 + c) * kHistBins + jb];
      }
    }
#pragma unroll
    for (int u = 0; u < kPlanBatch; ++u) {
      const int c = c0 + u;
      if (c < nc) {
        const float sc = fast_exp2((s_pm[c] - m) * rc.kk) * (1.0f / kFixScale);
        cnt += (float)(unsigned)(wb[u] >> 48);
        mass += (float)(wb[u] & kMassMask) * sc;
      }
    }
  }
  // N and Z (one reduction for both), and inclusive scans of counts and
  // masses from the top bin down.
  tcnt = wave_sum(tcnt);  // exact: < 2^24
  tmass = wave_sum(tmass);
  float C = wave_inclusive_sum(cnt), M = wave_inclusive_sum(mass);
  if (l == kWave - 1) {
    scratch[0][w] = tcnt;
    scratch[1][w] = tmass;
    wtot[0][w] = C;
    wtot[1][w] = M;
  }
  __syncthreads();
  float N = 0.0f, Z = 0.0f;
  for (int i = 0; i < kWaves; ++i) {
    N += scratch[0][i];
    Z += scratch[1][i];
    if (i < w) {
      C += wtot[0][i];
      M += wtot[1][i];
    }
  }
  const int k = a.top_k ? a.top_k[rc.b] : 0;
  const float tp = a.top_p ? a.top_p[rc.b] : 1.0f;
  const bool kA = k >= 1 && k < a.V && (float)k <= N;
  const bool pA = tp < 1.0f;
  // C and M do not decrease with the bin, so the first bin meeting a target
  // is the first set lane of the first wavefront whose ballot is not empty
  // (one LDS atomic per wavefront).
  const unsigned long long kb = __ballot(kA && C >= (float)k);
  if (l == 0 && kb) atomicMin(&first[0], w * kWave + __ffsll((unsigned long long)kb) - 1);
  __syncthreads();
  const int bk = kA ? first[0] : kRestBin;
  // Mass above bin bk (Z_lo) and through it (Z_hi): top-p's share is taken of
  // what top-k kept, which lies between the two.
  if (tid == 0) {
    zval[0] = 0.0f;
    zval[1] = Z;
  }
  __syncthreads();
  if (kA) {
    if (tid == bk - 1) zval[0] = M;
    if (tid == bk) zval[1] = M;
  } else if (tid == 0) {
    zval[0] = Z;
  }
  __syncthreads();
  if (pA) {
    const float tlo = tp * zval[0] * (1.0f - kPlanMargin);
    const float thi = tp * zval[1] * (1.0f + kPlanMargin);
    const unsigned long long lo = __ballot(M >= tlo), hi = __ballot(M >= thi);
    if (l == 0 && lo) atomicMin(&first[1], w * kWave + __ffsll((unsigned long long)lo) - 1);
    if (l == 0 && hi) atomicMin(&first[2], w * kWave + __ffsll((unsigned long long)hi) - 1);
  }
  __syncthreads();
  // Candidate range [rlo, rhi]. Top-k's own bin is always in it (the k-th
  // largest logit, and the share top-k keeps, are found among its tokens);
  // top-p's threshold lies between the bins its two targets reach.
  int rlo, rhi;
  if (!kA && !pA) {
    rlo = rhi = kKeepAll;  // nothing to drop
  } else if (!pA) {
    rlo = rhi = bk;
  } else if (!kA) {
    rlo = first[1];
    rhi = first[2];
  } else {
    rlo = min(first[1], bk);
    rhi = bk;
  }
  // Tokens above the range: the running count at bin rlo - 1.
  if (rlo >= 1 && rlo <= kRestBin && tid == rlo - 1) cabove = (int)C;
  __syncthreads();
  if (tid == 0) {
    a.plan[row * 2] = i32x4{a0, rlo, rhi, cabove};
    a.plan[row * 2 + 1] =
        i32x4{(kA ? 1 : 0) | (pA ? 2 : 0), k - cabove, __float_as_int(m), 0};
    a.tlist[atomicAdd(a.tcount, 1)] = (int)row;
  }
}

// Range test of a token's row bin rb against [rlo, rhi] (rhi = kRestBin:
// unbounded below the window).
__device__ __forceinline__ bool in_range(int rb, int rlo, int rhi) {
  return rb >= rlo && (rhi >= kRestBin || rb <= rhi);
}

// Row of list entry e of the truncated rows, or -1 past the list's end (the
// grids of the passes below cover every row; entries past the count exit).
__device__ __forceinline__ int64_t listed_row(const Args& a, int e) {
  return e < *a.tcount ? (int64_t)a.tlist[e] : -1;
}

// ---------------------------------------------------------------------------
// extract: (listed row, chunk) items, grid-stride (the grid is sized for the
// largest list; a workgroup takes items g, g + grid, ... below count x nc).
// ---------------------------------------------------------------------------
struct ExtractShared {
  int2 run[kWaves][kSegCap];  // each wavefront's candidates, in its own run
  float scratch[kWaves];
  int cnt[kWaves];
};

template <int DT, bool VP>
__device__ __forceinline__ void extract_item(const Args& a, int64_t row, int c,
                                             ExtractShared& sh);

template <int DT, bool VP>
__global__ __launch_bounds__(kThreads) void trunc_extract_kernel(Args a) {
  __shared__ ExtractShared sh;
  const int nc = a.nchunks;
  const int64_t items = (int64_t)*a.tcount * nc;
  for (int64_t x = blockIdx.x; x < items; x += gridDim.x) {
    const int e = (int)(x / nc);
    extract_item<DT, VP>(a, a.tlist[e], (int)(x - (int64_t)e * nc), sh);
  }
}

template <int DT, bool VP>
__device__ __forceinline__ void extract_item(const Args& a, int64_t row, int c,
                                             ExtractShared& sh) {
  const int tid = threadIdx.x, w = tid / kWave, l = tid % kWave;
  const int nc = a.nchunks;
  const int cstart = c * kChunk<DT>;
  u32x4 raw[kLoads];
  load_chunk<DT, VP>(a.logits + row * a.V * Dt<DT>::kBytes, cstart, a.V, tid, raw);
  const int b = (int)(row / (a.K + 1));
  const float kk = kLog2e / a.temperature[b];
  const i32x4 p0 = a.plan[row * 2], p1 = a.plan[row * 2 + 1];
  const int a0 = p0.x, rlo = p0.y, rhi = p0.z;
  const float m = __int_as_float(p1.z);
  float above = 0.0f;
  // Candidates are compacted per wavefront as they are found: a ballot per
  // element gives each finding lane its place after the wavefront's earlier
  // finds (element by element, lanes in order), in the wavefront's LDS run.
  // A run past kSegCap is not stored; the chunk then overflows its segment
  // (which holds at most kSegCap) and the row is selected by re-scanning it.
  int n = 0;  // wavefront-uniform
  int2* run = sh.run[w];
#pragma unroll
  for (int it = 0; it < kLoads; ++it)
#pragma unroll
    for (int k = 0; k < kVec<DT>; ++k) {
      const float v = elem<DT>(raw[it], k);
      const bool fin = v > kNegInf;
      const int rb = abs_bin(v, kk) - a0;
      if (fin && rb < rlo) above += fast_exp2((v - m) * kk);
      keep_here(above);
      const bool inr = fin && in_range(rb, rlo, rhi);
      const unsigned long long hit = __ballot(inr);
      if (inr) {
        const int p = n + lanes_below(hit);
        if (p < kSegCap)
          run[p] = int2{__float_as_int(v), elem_index<DT, VP>(cstart, tid, it, k)};
      }
      n += __popcll(hit);
    }
  above = wave_sum(above);
  if (l == 0) {
    sh.scratch[w] = above;
    sh.cnt[w] = n;
  }
  __syncthreads();
  // The runs go to this (row, chunk)'s own segment of the list in wavefront
  // order. A segment that would overflow is not written (its count says so).
  int base = 0, tot = 0;
  float sum = 0.0f;
#pragma unroll
  for (int i = 0; i < kWaves; ++i) {
    const int ci = sh.cnt[i];
    base += (i < w) ? ci : 0;
    tot += ci;
    sum += sh.scratch[i];
  }
  if (tid == 0) {
    a.tpart[row * nc + c] = sum;
    a.ccount[row * nc + c] = tot;
  }
  if (tot <= a.segcap) {
    int2* out = a.cand + (row * nc + c) * a.segcap + base;
    for (int p = l; p < n; p += kWave) out[p] = run[p];
  }
  __syncthreads();  // the runs and counts are reused by the next item
}

// ---------------------------------------------------------------------------
// select: one workgroup per listed row.
// ---------------------------------------------------------------------------
struct SelShared {
  unsigned key[kCandCap];  // candidate keys (fkey of the logit)
  unsigned char chunk[kCandCap];  // the chunk each candidate lies in
  int pre[kMaxChunks + 1];  // exclusive prefix of the chunks' candidate counts
  unsigned cnt[256];
  float mass[256];
  float csum[kMaxChunks];
  float scratch[kWaves];
  int iscr[2][kWaves];
  int digit;
  float carry;
  unsigned minkey;
};

// Candidate keys of a row: from LDS when they fit, else by re-reading the row
// and filtering it by the plan's range (exact, one pass over the row per
// call). f(key, list position or token index).
template <int DT, bool VP>
struct CandSource {
  // (fields by value: taking the kernel argument's address would place the
  // whole argument block in scratch memory)
  const unsigned char* rowp;
  int V, nchunks;
  SelShared* sh;
  int n, a0, rlo, rhi;
  float kk;
  bool lds;  // the candidates are in sh->key (else: re-scan the row)
  __device__ __forceinline__ bool in_lds() const { return lds; }
  template <typename F>
  __device__ __forceinline__ void each(F f) const {
    const int tid = threadIdx.x;
    if (in_lds()) {
      for (int i = tid; i < n; i += kThreads) f(sh->key[i], i);
      return;
    }
    for (int c = 0; c < nchunks; ++c) {
      const int cstart = c * kChunk<DT>;
      u32x4 raw[kLoads];
      load_chunk<DT, VP, false>(rowp, cstart, V, tid, raw);
#pragma unroll
      for (int it = 0; it < kLoads; ++it)
#pragma unroll
        for (int k = 0; k < kVec<DT>; ++k) {
          const float v = elem<DT>(raw[it], k);
          if (v > kNegInf && in_range(abs_bin(v, kk) - a0, rlo, rhi))
            f(fkey(v), elem_index<DT, VP>(cstart, tid, it, k));
        }
    }
  }
};

// Wavefront 0 scans the 256 digit buckets from digit 255 down (lane L holds
// digits 255-4L .. 252-4L) and leaves in sh.digit the first digit whose
// running total reaches t, in sh.carry the total of the digits above it
// (sh.digit = -1 when the buckets sum to less than t).
__device__ __forceinline__ void scan_digits(SelShared& sh, float t, bool by_mass) {
  const int tid = threadIdx.x;
  if (tid < kWave) {
    float v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int dg = 255 - 4 * tid - q;
      v[q] = by_mass ? sh.mass[dg] : (float)sh.cnt[dg];
    }
    const float lane = v[0] + v[1] + v[2] + v[3];
    const float inc = wave_inclusive_sum(lane);
    const unsigned long long hit = __ballot(inc >= t);
    if (hit) {
      const int L = __ffsll((unsigned long long)hit) - 1;
      if (tid == L) {
        float run = inc - lane;
        int q = 0;
        for (; q < 3; ++q) {
          if (run + v[q] >= t) break;
          run += v[q];
        }
        sh.digit = 255 - 4 * L - q;
        sh.carry = run;
      }
    } else if (tid == 0) {
      sh.digit = -1;
      sh.carry = 0.0f;
    }
  }
  __syncthreads();
}

// Radix digits below a common prefix: the candidates' keys agree on their
// top (32 - nbits) bits (prefix); selection walks the remaining bits in
// digits of up to 8 bits, so that no round puts every candidate in one
// bucket.
struct KeySpan {
  unsigned prefix;
  int nbits;
};

template <typename Src>
__device__ KeySpan key_span(const Src src, SelShared& sh) {
  const int tid = threadIdx.x, w = tid / kWave, l = tid % kWave;
  int lo = INT_MAX, hi = INT_MIN;  // keys as order-preserving signed ints
  src.each([&](unsigned key, int) {
    const int s = (int)(key ^ 0x80000000u);
    lo = min(lo, s);
    hi = max(hi, s);
  });
  lo = wave_min_i(lo);
  hi = wave_max_i(hi);
  if (l == 0) {
    sh.iscr[0][w] = lo;
    sh.iscr[1][w] = hi;
  }
  __syncthreads();
  for (int i = 0; i < kWaves; ++i) {
    lo = min(lo, sh.iscr[0][i]);
    hi = max(hi, sh.iscr[1][i]);
  }
  __syncthreads();
  const unsigned klo = (unsigned)lo ^ 0x80000000u, khi = (unsigned)hi ^ 0x80000000u;
  KeySpan ks;
  ks.nbits = (klo == khi) ? 0 : 32 - __clz((int)(klo ^ khi));
  ks.prefix = ks.nbits == 32 ? 0u : (klo >> ks.nbits) << ks.nbits;
  return ks;
}

// Key of the kth largest candidate (1-based; kth <= the candidate count).
template <typename Src>
__device__ unsigned select_kth(const Src src, SelShared& sh, KeySpan ks, int kth) {
  const int tid = threadIdx.x;
  unsigned prefix = ks.prefix;
  float need = (float)kth;
  for (int rem = ks.nbits; rem > 0;) {
    const int wd = min(8, rem);
    rem -= wd;
    const unsigned mask = (rem + wd >= 32) ? 0u : (~0u << (rem + wd));  // bits above
    sh.cnt[tid] = 0;
    __syncthreads();
    src.each([&](unsigned key, int) {
      if ((key & mask) == prefix)
        atomicAdd(&sh.cnt[(key >> rem) & ((1u << wd) - 1)], 1u);
    });
    __syncthreads();
    scan_digits(sh, need, false);
    const int dg = sh.digit < 0 ? 0 : sh.digit;
    need -= sh.carry;
    prefix |= (unsigned)dg << rem;
    __syncthreads();
  }
  return prefix;
}

// Largest key K >= kmin such that the candidates with keys in [K, inf) carry
// at least t of probability; the smallest candidate key >= kmin when rounding
// leaves the candidates short of t.
template <typename Src>
__device__ unsigned select_mass(const Src src, SelShared& sh, KeySpan ks, float t,
                                unsigned kmin, float m, float kk) {
  const int tid = threadIdx.x;
  unsigned prefix = ks.prefix;
  bool found = true;
  for (int rem = ks.nbits; rem > 0 && found;) {
    const int wd = min(8, rem);
    rem -= wd;
    const unsigned mask = (rem + wd >= 32) ? 0u : (~0u << (rem + wd));
    sh.mass[tid] = 0.0f;
    __syncthreads();
    src.each([&](unsigned key, int) {
      if (key >= kmin && (key & mask) == prefix)
        atomicAdd(&sh.mass[(key >> rem) & ((1u << wd) - 1)],
                  fast_exp2((fkey_inv(key) - m) * kk));
    });
    __syncthreads();
    scan_digits(sh, t, true);
    if (sh.digit < 0) {
      found = false;
    } else {
      t -= sh.carry;
      prefix |= (unsigned)sh.digit << rem;
    }
    __syncthreads();
  }
  if (found) return prefix;
  if (tid == 0) sh.minkey = 0xffffffffu;
  __syncthreads();
  src.each([&](unsigned key, int) {
    if (key >= kmin) atomicMin(&sh.minkey, key);
  });
  __syncthreads();
  return sh.minkey;
}

template <int DT, bool VP>
__global__ __launch_bounds__(kThreads) void trunc_select_kernel(Args a) {
  __shared__ SelShared sh;
  const int tid = threadIdx.x, w = tid / kWave, l = tid % kWave;
  // One workgroup per listed row; workgroups past the list's end leave at
  // once (they hold this kernel's large LDS block only for one load).
  const int64_t row = listed_row(a, blockIdx.x);
  if (row < 0) return;
  const int nc = a.nchunks;
  const i32x4 p0 = a.plan[row * 2], p1 = a.plan[row * 2 + 1];
  int cc = 0;
  float tb = 0.0f;
  f32x4 pv = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  if (tid < nc) {
    cc = a.ccount[row * nc + tid];
    tb = a.tpart[row * nc + tid];
    pv = a.partials[row * nc + tid];
  }
  const int b = (int)(row / (a.K + 1));
  const float kk = kLog2e / a.temperature[b];
  const int mode = p1.x, krem = p1.y;
  const float m = __int_as_float(p1.z);
  for (int c = tid + kThreads; c < nc; c += kThreads) tb += a.tpart[row * nc + c];
  // Probability above the range: every token there is kept.
  const float base = block_sum(tb, sh.scratch);
  if (mode == 0) {
    if (tid == 0) a.tinfo[row] = f32x4{kNegInf, base, 1.0f, 0.0f};
    return;
  }
  // Exclusive prefix of the chunks' candidate counts (nc <= kThreads here;
  // more chunks than threads, or an overflowing segment, take the re-scan).
  const bool over = nc > kThreads || cc > a.segcap;
  const int inc = (int)wave_inclusive_sum((float)cc);
  if (l == kWave - 1) sh.iscr[0][w] = inc;
  __syncthreads();
  int wb = 0, tot = 0;
  for (int i = 0; i < kWaves; ++i) {
    if (i < w) wb += sh.iscr[0][i];
    tot += sh.iscr[0][i];
  }
  if (tid < nc) sh.pre[tid] = wb + inc - cc;
  if (tid == 0) sh.pre[nc < kThreads ? nc : kThreads] = tot;
  const int anyover = __syncthreads_or(over);
  const bool lds = !anyover && tot <= kCandCap;
  const int n = tot;
  if (lds) {
    // Entry f of the list lies in chunk c with pre[c] <= f < pre[c+1].
    const int2* seg = a.cand + row * nc * a.segcap;
    constexpr int kU = 16;  // loads in flight per thread: 4,096 candidates in one round trip
    for (int f0 = 0; f0 < n; f0 += kU * kThreads) {
      int2 ev[kU];
      int ch[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int f = f0 + u * kThreads + tid;
        ev[u] = int2{0, 0};
        ch[u] = 0;
        if (f < n) {
          int lo = 0, hi = nc - 1;
          while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (sh.pre[mid] <= f) lo = mid;
            else hi = mid - 1;
          }
          ch[u] = lo;
          ev[u] = seg[(int64_t)lo * a.segcap + (f - sh.pre[lo])];
        }
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int f = f0 + u * kThreads + tid;
        if (f < n) {
          sh.key[f] = fkey(__int_as_float(ev[u].x));
          sh.chunk[f] = (unsigned char)ch[u];
        }
      }
    }
  }
  for (int c = tid; c < nc; c += kThreads) sh.csum[c] = 0.0f;
  __syncthreads();
  const CandSource<DT, VP> src{a.logits + row * a.V * Dt<DT>::kBytes, a.V, nc, &sh,
                               n, p0.x, p0.y, p0.z, kk, lds};
  const KeySpan ks = key_span(src, sh);
  unsigned kmin = 0;
  if (mode & 1) kmin = select_kth(src, sh, ks, krem);
  unsigned key = kmin;
  if (mode & 2) {
    // top-p's share is of what top-k kept: with top-k, base plus the
    // candidates at or above kmin (everything below the range is below the
    // k-th largest); without, the whole row (from the stream partials).
    float zk = 0.0f;
    if (mode & 1) {
      src.each([&](unsigned k2, int) {
        if (k2 >= kmin) zk += fast_exp2((fkey_inv(k2) - m) * kk);
      });
      zk = base + block_sum(zk, sh.scratch);
    } else {
      zk = (tid < nc) ? pv.y * fast_exp2((pv.x - m) * kk) : 0.0f;
      for (int c = tid + kThreads; c < nc; c += kThreads) {
        const f32x4 p = a.partials[row * nc + c];
        zk += p.y * fast_exp2((p.x - m) * kk);
      }
      zk = block_sum(zk, sh.scratch);
    }
    const float t = a.top_p[b] * zk - base;
    if (t > 0.0f) {
      key = select_mass(src, sh, ks, t, kmin, m, kk);
    } else {
      // The range is chosen so that this does not happen (the share above
      // it stays below top_p); keep the top candidate group if it does.
      if (tid == 0) sh.minkey = 0;
      __syncthreads();
      src.each([&](unsigned k2, int) { atomicMax(&sh.minkey, k2); });
      __syncthreads();
      key = sh.minkey;
    }
  }
  // Kept candidates: their probability, per chunk. In LDS the list is grouped
  // by chunk: each thread sums a contiguous run and adds it to its chunk when
  // the chunk changes. The re-scan adds token by token.
  if (lds) {
    const int per = (n + kThreads - 1) / kThreads;
    const int f0 = tid * per, f1 = min(n, f0 + per);
    int cur = -1;
    float run = 0.0f;
    for (int f = f0; f < f1; ++f) {
      const int ch = sh.chunk[f];
      if (ch != cur) {
        if (cur >= 0 && run != 0.0f) atomicAdd(&sh.csum[cur], run);
        cur = ch;
        run = 0.0f;
      }
      const unsigned k2 = sh.key[f];
      if (k2 >= key) run += fast_exp2((fkey_inv(k2) - m) * kk);
    }
    if (cur >= 0 && run != 0.0f) atomicAdd(&sh.csum[cur], run);
  } else {
    src.each([&](unsigned k2, int i) {
      if (k2 >= key) atomicAdd(&sh.csum[i / kChunk<DT>], fast_exp2((fkey_inv(k2) - m) * kk));
    });
  }
  __syncthreads();
  float kept = 0.0f;
  for (int c = tid; c < nc; c += kThreads) {
    const float t = a.tpart[row * nc + c] + sh.csum[c];
    a.tpart[row * nc + c] = t;
    kept += t;
  }
  kept = block_sum(kept, sh.scratch);
  if (tid == 0) a.tinfo[row] = f32x4{fkey_inv(key), kept, 1.0f, 0.0f};
}

template <int DT, bool VP>
int launch_t(const Args& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.B * (a.K + 1);
  hipLaunchKernelGGL(trunc_plan_kernel, dim3((unsigned)rows), dim3(kThreads), 0, s, a);
  int rc = check_launch("truncation plan");
  if (rc != SS_OK) return rc;
  // Enough workgroups to fill the chip several times over; each takes the
  // items of the listed rows in turn.
  const int64_t grid = std::min<int64_t>(rows * a.nchunks, kExtractGrid);
  hipLaunchKernelGGL((trunc_extract_kernel<DT, VP>), dim3((unsigned)grid),
                     dim3(kThreads), 0, s, a);
  rc = check_launch("truncation extract");
  if (rc != SS_OK) return rc;
  hipLaunchKernelGGL((trunc_select_kernel<DT, VP>), dim3((unsigned)rows),
                     dim3(kThreads), 0, s, a);
  return check_launch("truncation select");
}

}  // namespace

int launch_truncation(const Args& a, bool f32, bool vp, hipStream_t s) {
  return f32 ? (vp ? launch_t<SS_DTYPE_F32, true>(a, s)
                   : launch_t<SS_DTYPE_F32, false>(a, s))
             : (vp ? launch_t<SS_DTYPE_BF16, true>(a, s)
                   : launch_t<SS_DTYPE_BF16, false>(a, s));
}

}  // namespace specsam
