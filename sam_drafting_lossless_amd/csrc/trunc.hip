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
// digit, would cost several passes over HBM. Here the row is read once:
//   stream  (stream.hip, truncated rows only) counts each chunk's logits, and
//           sums their probability, in a 256-bin window histogram on a grid
//           shared by all chunks of the row (1/8 octave of probability per
//           bin, 32 octaves below the chunk max); picks a band of bins from
//           its own histogram (its top bins down to its own k-th largest
//           logit for top-k; a few bins around its own top_p point for top-p
//           alone), copies the band's logits to the chunk's segment and sums
//           the probability of its tokens above the band;
//   select  (one 1024-thread workgroup per row) merges the row's chunk
//           histograms, scans them from the top and picks the bin range that
//           must hold the threshold (with a margin for the histogram's
//           rounding); takes the candidates (the tokens in the range) and the
//           exact probability above the range from each chunk's band when the
//           band holds the range, else by re-reading that chunk; finds the
//           exact threshold among the candidates by radix selection on
//           order-preserving keys (8-bit digits, LDS histograms of counts for
//           top-k and of probability for top-p); and leaves each chunk's kept
//           probability.
// The finalize kernel then judges and draws with the per-chunk kept sums and
// the threshold. Selection first finds the bits all candidate keys share and
// radix-walks only the bits below them, so that no round piles every
// candidate into one LDS bucket. A row with more than kCandCap candidates is
// selected by walking its chunks' tokens again in each round (from the
// segments, or the logits for chunks whose band misses): exact, but slower.
// The sums that reach the outputs are taken in a fixed order.
#include <algorithm>

#include "verify_common.h"

namespace specsam {
namespace {

constexpr float kPlanMargin = 1e-4f;  // relative slack for histogram rounding
constexpr int kSelThreads = 512;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kPlanGroups = kSelThreads / kHistBins;  // chunk groups of the merge
constexpr int kPlanBatch = 10;  // histogram words a thread requests at once (one batch
                                // for V = 151,936 fp32: 19 chunks over two groups)
static_assert(kMaxChunks <= kHistBins, "the chunk prefix uses the first 4 wavefronts");

// Row-level activity of truncation; the same test as the stream pass.
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

struct SelShared {
  unsigned key[kCandCap];  // candidate keys (fkey of the logit), a run per chunk
  // per chunk: window start bin, finite count, max, weight sum (relative to
  // its max), packed band, band logits, weight above the band (relative to
  // its max); candidates found, exclusive prefix of those, weight above the
  // range and kept weight (relative to the row max)
  int ca[kMaxChunks];
  int cnf[kMaxChunks];
  float cpm[kMaxChunks];
  float cps[kMaxChunks];
  int cband[kMaxChunks];
  int cn[kMaxChunks];
  float cab[kMaxChunks];
  int ccnt[kMaxChunks];
  int cbeg[kMaxChunks];      // where the chunk's run of keys starts
  float cabove[kMaxChunks];
  float ckept[kMaxChunks];
  int miss[kMaxChunks];      // chunks whose band misses the range, in order
  int wcnt[kSelWaves];       // per-wavefront candidate counts of a re-read chunk
  int ncand;                 // keys placed (runs reserved) so far
  int over;                  // the runs would pass kCandCap
  int mbase;
  float pc[kPlanGroups][kHistBins];  // merge: each chunk group's count per row bin
  float pw[kPlanGroups][kHistBins];  // and weight
  unsigned cnt[256];
  float mass[256];
  float wtot[2][kSelWaves];
  float scratch[kSelWaves];
  int iscr[2][kSelWaves];
  int first[3];
  int cabove_n;
  float zval[2];
  int digit;
  float carry;
  unsigned minkey;
};

__device__ __forceinline__ float block_sum(float v, float* scratch) {
  const int tid = threadIdx.x, w = tid / kWave, l = tid % kWave;
  v = wave_sum(v);
  __syncthreads();
  if (l == 0) scratch[w] = v;
  __syncthreads();
  float t = 0.0f;
  for (int i = 0; i < kSelWaves; ++i) t += scratch[i];
  return t;
}

// Every logit of chunk c of a row, read by one wavefront, 8 16-byte loads
// per lane in flight: f(value) in a fixed order, on every lane the same
// number of times (past the row's end with -inf), so f may use ballots.
template <int DT, bool VP, typename F>
__device__ __forceinline__ void wave_chunk_each(const unsigned char* rowp, int c, int V,
                                                F f) {
  constexpr unsigned kNegInfWord = DT == SS_DTYPE_F32 ? 0xff800000u : 0xff80ff80u;
  constexpr int kU = 8;
  const int l = threadIdx.x % kWave;
  const int cstart = c * kChunk<DT>;
  const int rem = min(kChunk<DT>, V - cstart);
  if constexpr (VP) {
    // (V is a multiple of the vector width on this path)
    const u32x4* p = reinterpret_cast<const u32x4*>(rowp + (int64_t)cstart * Dt<DT>::kBytes);
    const int nv = rem / kVec<DT>;
    for (int v0 = 0; v0 < nv; v0 += kU * kWave) {
      u32x4 r[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int vi = v0 + u * kWave + l;
        r[u] = vi < nv ? __builtin_nontemporal_load(p + vi)
                       : u32x4{kNegInfWord, kNegInfWord, kNegInfWord, kNegInfWord};
      }
#pragma unroll
      for (int u = 0; u < kU; ++u)
#pragma unroll
        for (int k = 0; k < kVec<DT>; ++k) f(elem<DT>(r[u], k));
    }
  } else {
    for (int e0 = 0; e0 < rem; e0 += kU * kWave) {
      float r[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) {
        const int e = e0 + u * kWave + l;
        r[u] = e < rem ? load_one<DT>(rowp, (int64_t)cstart + e) : kNegInf;
      }
#pragma unroll
      for (int u = 0; u < kU; ++u) f(r[u]);
    }
  }
}

// Chunk c of a row read by the whole workgroup in one round trip: element
// i of thread t is token c * kChunk + (t + i * kSelThreads) (16-byte path:
// vector t + u * kSelThreads, element k, in that order); -inf past the row.
template <int DT>
constexpr int kBlkElems = kChunk<DT> / kSelThreads;

template <int DT, bool VP>
__device__ __forceinline__ void block_chunk_load(const unsigned char* rowp, int c, int V,
                                                 float (&v)[kBlkElems<DT>]) {
  const int tid = threadIdx.x;
  const int cstart = c * kChunk<DT>;
  const int rem = min(kChunk<DT>, V - cstart);
  if constexpr (VP) {
    constexpr int kNV = kBlkElems<DT> / kVec<DT>;
    const u32x4* p = reinterpret_cast<const u32x4*>(rowp + (int64_t)cstart * Dt<DT>::kBytes);
    const int nv = rem / kVec<DT>;
    u32x4 r[kNV];
#pragma unroll
    for (int u = 0; u < kNV; ++u) {
      const int vi = tid + u * kSelThreads;
      r[u] = vi < nv ? __builtin_nontemporal_load(p + vi) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kNV; ++u)
#pragma unroll
      for (int k = 0; k < kVec<DT>; ++k)
        v[u * kVec<DT> + k] = (tid + u * kSelThreads < nv) ? elem<DT>(r[u], k) : kNegInf;
  } else {
#pragma unroll
    for (int i = 0; i < kBlkElems<DT>; ++i) {
      const int e = tid + i * kSelThreads;
      v[i] = e < rem ? load_one<DT>(rowp, (int64_t)cstart + e) : kNegInf;
    }
  }
}

// A row's tokens at or above the bottom of its range [rlo, rhi], chunk by
// chunk. Fields by value: taking the kernel argument's address would place
// the whole argument block in scratch memory.
template <int DT, bool VP>
struct RowSrc {
  const unsigned char* rowp;  // the row's logits
  const float* seg;           // the row's band segments
  int V, nc, segcap;
  int a0, rlo, rhi;
  float m, kk, ns;
  SelShared* sh;
  bool lds;  // the candidates are in sh->key (else: walk the chunks again)
  int n;     // candidates
  // The range on the product t = l * ns (see band_t): a token lies above
  // it when t < t_lo, in it when t_lo <= t < t_hi (t_hi = +inf for a range
  // open below the window; -inf, whose product is +inf, and NaN lie in
  // neither).
  float t_lo, t_hi;

  __device__ __forceinline__ bool above(float v) const { return v * ns < t_lo; }
  __device__ __forceinline__ bool cand(float v) const {
    const float t = v * ns;
    return (t >= t_lo) & (t < t_hi);
  }

  // How chunk c's tokens at or above the range's bottom are found: kNone
  // (it has none: its max lies below the range), kBand (its band holds
  // them all), kReread (its band misses part of the range).
  static constexpr int kNone = 0, kBand = 1, kReread = 2;
  __device__ __forceinline__ int source(int c) const {
    const int sc = sh->ca[c] - a0;  // the chunk's window starts at row bin sc
    if (rhi < kRestBin && rhi < sc) return kNone;
    const int bd = sh->cband[c];
    const int blo = bd & 0xffff, bhi = bd >> 16;
    const bool covered = blo <= bhi && blo + sc <= max(rlo, sc) &&
                         (bhi >= kRestBin || (rhi < kRestBin && rhi <= bhi + sc));
    return covered ? kBand : kReread;
  }

  // Wavefront-wide: chunk c's segment (a kBand chunk) into r, lane l holding
  // entries l, l + 64, ... (-inf past its end); returns the number of
  // wavefront rows in use. The whole segment is requested at once.
  static constexpr int kU = kSegCap / kWave;
  __device__ __forceinline__ int band_load(int c, float (&r)[kU]) const {
    const int l = threadIdx.x % kWave;
    const int cn = min(sh->cn[c], segcap);
    const float* sp = seg + (int64_t)c * segcap;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = u * kWave + l;
      r[u] = i < cn ? sp[i] : kNegInf;
    }
    return (cn + kWave - 1) / kWave;
  }

  // Wavefront-wide: f(v) for every logit of chunk c that may lie at or above
  // the range (its band's, or all of its logits when the band misses).
  template <typename F>
  __device__ __forceinline__ void chunk(int c, F f) const {
    const int src = source(c);
    if (src == kNone) return;
    if (src == kBand) {
      float r[kU];
      const int nu = band_load(c, r);
#pragma unroll
      for (int u = 0; u < kU; ++u)
        if (u < nu) f(r[u]);
      return;
    }
    wave_chunk_each<DT, VP>(rowp, c, V, f);
  }

  // f(key) for every candidate (each round of the selection).
  template <typename F>
  __device__ __forceinline__ void each(F f) const {
    const int tid = threadIdx.x, w = tid / kWave;
    if (lds) {
      for (int i = tid; i < n; i += kSelThreads) f(sh->key[i]);
      return;
    }
    for (int c = w; c < nc; c += kSelWaves)
      chunk(c, [&](float v) {
        if (cand(v)) f(fkey(v));
      });
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
__device__ __forceinline__ KeySpan key_span(const Src& src, SelShared& sh) {
  const int tid = threadIdx.x, w = tid / kWave, l = tid % kWave;
  int lo = INT_MAX, hi = INT_MIN;  // keys as order-preserving signed ints
  src.each([&](unsigned key) {
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
  for (int i = 0; i < kSelWaves; ++i) {
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
__device__ __forceinline__ unsigned select_kth(const Src& src, SelShared& sh, KeySpan ks,
                                             int kth) {
  const int tid = threadIdx.x;
  unsigned prefix = ks.prefix;
  float need = (float)kth;
  for (int rem = ks.nbits; rem > 0;) {
    const int wd = min(8, rem);
    rem -= wd;
    const unsigned mask = (rem + wd >= 32) ? 0u : (~0u << (rem + wd));  // bits above
    if (tid < 256) sh.cnt[tid] = 0;
    __syncthreads();
    src.each([&](unsigned key) {
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
__device__ __forceinline__ unsigned select_mass(const Src& src, SelShared& sh, KeySpan ks,
                                              float t, unsigned kmin, float m, float kk) {
  const int tid = threadIdx.x;
  unsigned prefix = ks.prefix;
  bool found = true;
  for (int rem = ks.nbits; rem > 0 && found;) {
    const int wd = min(8, rem);
    rem -= wd;
    const unsigned mask = (rem + wd >= 32) ? 0u : (~0u << (rem + wd));
    if (tid < 256) sh.mass[tid] = 0.0f;
    __syncthreads();
    src.each([&](unsigned key) {
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
  src.each([&](unsigned key) {
    if (key >= kmin) atomicMin(&sh.minkey, key);
  });
  __syncthreads();
  return sh.minkey;
}

// ---------------------------------------------------------------------------
// select: one workgroup per row (rows that are not truncated leave at once).
// ---------------------------------------------------------------------------
template <int DT, bool VP>
__global__ __launch_bounds__(kSelThreads) void trunc_select_kernel(Args a) {
  __shared__ SelShared sh;
  const int tid = threadIdx.x, w = tid / kWave, l = tid % kWave;
  // Blocks take rows j-major (block x: sequence x mod B, row x div B): the
  // rows every sequence needs (row 0) are then consecutive blocks, which
  // the dispatcher spreads over all XCDs, rather than every (K+1)-th block.
  const int bx = blockIdx.x;
  const int64_t row = (int64_t)(bx % a.B) * (a.K + 1) + bx / a.B;
  const int nc = a.nchunks;
  const int64_t h0 = row * nc;
  // The chunk headers, partials and above-band weights are requested
  // together with the row's parameters (they are in bounds for every row;
  // an inactive row's are never used).
  i32x4 hh = i32x4{0, 0, 0, 0};
  f32x4 pv = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  float ab = 0.0f;
  if (tid < nc) {
    hh = a.hhdr[h0 + tid];
    pv = a.partials[h0 + tid];
    ab = a.tpart[h0 + tid];
  }
  const RowCtx rc = row_ctx(a, row);
  if (!rc.active) return;
  const float kk = rc.kk;
  if (tid < nc) {
    sh.ca[tid] = hh.x;
    sh.cnf[tid] = hh.y;
    sh.cband[tid] = hh.z;
    sh.cn[tid] = hh.w;
    sh.cpm[tid] = pv.x;
    sh.cps[tid] = pv.y;
    sh.cab[tid] = ab;
  }
  if (tid < 3) sh.first[tid] = kRestBin;
  if (tid == 0) {
    sh.cabove_n = 0;
    sh.ncand = 0;
    sh.over = 0;
  }
  __syncthreads();
  // Each wavefront's segments (wavefront w takes chunks w, w + kSelWaves,
  // ...), each requested one chunk ahead of its use, the first now, while
  // the plan below decides whether it is used. The loads take no branch (an
  // index past the segment's count is clamped into it and the entry masked
  // where it is used) and two buffers alternate, so that the wait for one
  // segment leaves the next in flight: a load behind a branch, or a
  // register copy of a loaded value, makes the compiler wait for every load
  // in flight.
  // A row whose segments all hold at most kSmallSegU wavefront rows (top-k's
  // bands) requests that many per segment, others all kSegU.
  constexpr int kSegU = kSegCap / kWave;
  constexpr int kSmallSegU = 2;
  using SmallSeg = std::integral_constant<int, kSmallSegU>;
  using FullSeg = std::integral_constant<int, kSegU>;
  int mcn = 0;
  for (int c = l; c < nc; c += kWave) mcn = max(mcn, min(sh.cn[c], a.segcap));
  const bool small_seg = wave_max_i(mcn) <= kSmallSegU * kWave;
  auto seg_issue = [&](auto nu, int c, bool banded, float (&r)[kSegU])
                       __attribute__((always_inline)) {
    const int cn = banded ? min(sh.cn[c], a.segcap) : 0;
    const float* sp = a.cand + (h0 + c) * a.segcap;
    const int last = max(cn, 1) - 1;
#pragma unroll
    for (int u = 0; u < decltype(nu)::value; ++u) r[u] = sp[min(u * kWave + l, last)];
    return cn;
  };
  float sa[kSegU], sb[kSegU];
  int na = 0;  // entries of sa in use
  if (w < nc) {
    const int bd = sh.cband[w];
    const bool banded = (bd & 0xffff) <= (bd >> 16);
    na = small_seg ? seg_issue(SmallSeg{}, w, banded, sa) : seg_issue(FullSeg{}, w, banded, sa);
  }
  // Row max m, finite count N and weight Z (relative to m): every wavefront
  // reduces the chunk values itself, in the same order.
  float m = kNegInf;
  for (int c = l; c < nc; c += kWave) m = fmaxf(m, sh.cpm[c]);
  m = wave_max(m);
  float tn = 0.0f, tz = 0.0f;
  for (int c = l; c < nc; c += kWave) {
    tn += (float)sh.cnf[c];
    tz += sh.cps[c] * fast_exp2((sh.cpm[c] - m) * kk);
  }
  const float N = wave_sum(tn);  // exact: < 2^24
  const float Z = wave_sum(tz);
  const float ns = bin_scale(kk);
  const int a0 = abs_bin_s(m, ns);
  // Merge: bin r of the row is bin r - (a_c - a0) of chunk c. Thread (g, r)
  // adds the chunks c = g (mod kPlanGroups), kPlanBatch words requested at
  // once; the groups' sums are added in group order.
  {
    const int r = tid % kHistBins, g = tid / kHistBins;
    float cnt = 0.0f, mass = 0.0f;
    for (int c0 = g; c0 < nc; c0 += kPlanGroups * kPlanBatch) {
      unsigned long long wb[kPlanBatch];
#pragma unroll
      for (int u = 0; u < kPlanBatch; ++u) {
        const int c = c0 + u * kPlanGroups;
        wb[u] = 0;
        if (c < nc) {
          const int jb = r - (sh.ca[c] - a0);
          if (jb >= 0 && jb < kHistBins) wb[u] = a.hist[(h0 + c) * kHistBins + jb];
        }
      }
#pragma unroll
      for (int u = 0; u < kPlanBatch; ++u) {
        const int c = c0 + u * kPlanGroups;
        if (c < nc) {
          const float sc = fast_exp2((sh.cpm[c] - m) * kk) * (1.0f / kFixScale);
          cnt += (float)(unsigned)(wb[u] >> 48);
          mass += (float)(wb[u] & kMassMask) * sc;
        }
      }
    }
    sh.pc[g][r] = cnt;
    sh.pw[g][r] = mass;
  }
  __syncthreads();
  // Thread r < 256 owns row bin r: inclusive scans of counts (C) and
  // weights (M) from the top bin down.
  const bool binT = tid < kHistBins;
  float C = 0.0f, M = 0.0f;
  if (binT) {
    for (int g = 0; g < kPlanGroups; ++g) {
      C += sh.pc[g][tid];
      M += sh.pw[g][tid];
    }
    C = wave_inclusive_sum(C);
    M = wave_inclusive_sum(M);
    if (l == kWave - 1) {
      sh.wtot[0][w] = C;
      sh.wtot[1][w] = M;
    }
  }
  __syncthreads();
  if (binT) {
    for (int i = 0; i < w; ++i) {
      C += sh.wtot[0][i];
      M += sh.wtot[1][i];
    }
  }
  const int k = a.top_k ? a.top_k[rc.b] : 0;
  const float tp = a.top_p ? a.top_p[rc.b] : 1.0f;
  const bool kA = k >= 1 && k < a.V && (float)k <= N;
  const bool pA = tp < 1.0f;
  // C and M do not decrease with the bin, so the first bin meeting a target
  // is the first set lane of the first wavefront whose ballot is not empty
  // (one LDS atomic per wavefront).
  if (binT) {
    const unsigned long long kb = __ballot(kA && C >= (float)k);
    if (l == 0 && kb) atomicMin(&sh.first[0], w * kWave + __ffsll((unsigned long long)kb) - 1);
  }
  if (tid == 0) {
    sh.zval[0] = 0.0f;
    sh.zval[1] = Z;
  }
  __syncthreads();
  const int bk = kA ? sh.first[0] : kRestBin;
  // Weight above bin bk (Z_lo) and through it (Z_hi): top-p's share is taken
  // of what top-k kept, which lies between the two.
  if (kA && binT) {
    if (tid == bk - 1) sh.zval[0] = M;
    if (tid == bk) sh.zval[1] = M;
  } else if (tid == 0) {
    sh.zval[0] = Z;
  }
  __syncthreads();
  if (pA && binT) {
    const float tlo = tp * sh.zval[0] * (1.0f - kPlanMargin);
    const float thi = tp * sh.zval[1] * (1.0f + kPlanMargin);
    const unsigned long long lo = __ballot(M >= tlo), hi = __ballot(M >= thi);
    if (l == 0 && lo) atomicMin(&sh.first[1], w * kWave + __ffsll((unsigned long long)lo) - 1);
    if (l == 0 && hi) atomicMin(&sh.first[2], w * kWave + __ffsll((unsigned long long)hi) - 1);
  }
  __syncthreads();
  const int mode = (kA ? 1 : 0) | (pA ? 2 : 0);
  if (mode == 0) {
    // Nothing is dropped (k at least the finite count, no top-p).
    if (tid < nc) a.tpart[h0 + tid] = sh.cps[tid] * fast_exp2((sh.cpm[tid] - m) * kk);
    if (tid == 0) a.tinfo[row] = f32x4{kNegInf, Z, 1.0f, 0.0f};
    return;
  }
  // Candidate range [rlo, rhi]. Top-k's own bin is always in it (the k-th
  // largest logit, and the share top-k keeps, are found among its tokens);
  // top-p's threshold lies between the bins its two targets reach.
  int rlo, rhi;
  if (!pA) {
    rlo = rhi = bk;
  } else if (!kA) {
    rlo = sh.first[1];
    rhi = sh.first[2];
  } else {
    rlo = min(sh.first[1], bk);
    rhi = bk;
  }
  // Tokens above the range: the running count at bin rlo - 1.
  if (rlo >= 1 && rlo <= kRestBin && tid == rlo - 1) sh.cabove_n = (int)C;
  __syncthreads();
  const int krem = k - sh.cabove_n;
  RowSrc<DT, VP> src{a.logits + row * a.V * Dt<DT>::kBytes,
                     a.cand + h0 * a.segcap,
                     a.V, nc, a.segcap, a0, rlo, rhi, m, kk, ns, &sh, false, 0,
                     (float)(a0 + rlo),
                     rhi >= kRestBin ? INFINITY : (float)(a0 + rhi + 1)};
  using Src = RowSrc<DT, VP>;
  // Chunks whose band misses the range, listed in chunk order (nc <= 256:
  // the first four wavefronts).
  {
    const bool miss = tid < nc && src.source(tid) == Src::kReread;
    const unsigned long long mb = __ballot(miss);
    if (l == 0 && w < kHistBins / kWave) sh.iscr[1][w] = __popcll(mb);
    __syncthreads();
    int at = 0;
    for (int i = 0; i < w && i < kHistBins / kWave; ++i) at += sh.iscr[1][i];
    if (miss) sh.miss[at + lanes_below(mb)] = tid;
  }
  int nmiss = 0;
  for (int i = 0; i < kHistBins / kWave; ++i) nmiss += sh.iscr[1][i];
  __syncthreads();
  // Each chunk's candidates, as one run of keys in LDS (its place taken with
  // one LDS atomic; within the run, in the order met), and its weight above
  // the range: from its band (a wavefront per chunk), or by the whole
  // workgroup re-reading it. Runs that would pass kCandCap are not stored
  // (the selection then walks the chunks in each round).
  auto above_w = [&](float v) { return src.above(v) ? fast_exp2((v - m) * kk) : 0.0f; };
  auto is_cand = [&](float v) { return src.cand(v); };
  auto put = [&](float v, int& pos) {
    const bool in = is_cand(v);
    const unsigned long long hit = __ballot(in);
    if (in) sh.key[pos + lanes_below(hit)] = fkey(v);
    pos += __popcll(hit);
  };
  // The candidates and the weight above the range of chunk c from its
  // segment sg of cn entries (a kBand chunk), or nothing (kNone).
  auto take_band = [&](auto nu_max, int c, const float (&sg)[kSegU], int cn)
                       __attribute__((always_inline)) {
    const int sk = src.source(c);
    if (sk == Src::kReread) return;
    float above = 0.0f;
    int cnt = 0, at = 0;  // wavefront-uniform
    if (sk == Src::kBand) {
      const int nu = (cn + kWave - 1) / kWave;
#pragma unroll
      for (int u = 0; u < decltype(nu_max)::value; ++u)
        if (u < nu) {
          const float v = u * kWave + l < cn ? sg[u] : kNegInf;
          above += above_w(v);
          cnt += __popcll(__ballot(is_cand(v)));
        }
      if (l == 0) at = atomicAdd(&sh.ncand, cnt);
      at = __builtin_amdgcn_readfirstlane(at);
      if (at + cnt <= kCandCap) {
        int pos = at;
#pragma unroll
        for (int u = 0; u < decltype(nu_max)::value; ++u)
          if (u < nu) put(u * kWave + l < cn ? sg[u] : kNegInf, pos);
      } else if (l == 0) {
        sh.over = 1;
      }
      above = wave_sum(above) + sh.cab[c] * fast_exp2((sh.cpm[c] - m) * kk);
    }
    if (l == 0) {
      sh.ccnt[c] = cnt;
      sh.cbeg[c] = at;
      sh.cabove[c] = above;
    }
  };
  // The next segment's request (a chunk past the last, or one without a
  // band, requests the wavefront's own first segment and uses none of it).
  auto next_seg = [&](auto nu, int c, float (&r)[kSegU]) __attribute__((always_inline)) {
    const bool band = c < nc && src.source(c) == Src::kBand;
    return seg_issue(nu, band ? c : w, band, r);
  };
  auto gather = [&](auto nu) __attribute__((always_inline)) {
    for (int c = w; c < nc; c += 2 * kSelWaves) {
      const int nb = next_seg(nu, c + kSelWaves, sb);
      take_band(nu, c, sa, na);
      if (c + kSelWaves >= nc) break;
      na = next_seg(nu, c + 2 * kSelWaves, sa);
      take_band(nu, c + kSelWaves, sb, nb);
    }
  };
  if (small_seg)
    gather(SmallSeg{});
  else
    gather(FullSeg{});
  for (int i = 0; i < nmiss; ++i) {
    const int c = sh.miss[i];
    float v[kBlkElems<DT>];
    block_chunk_load<DT, VP>(src.rowp, c, a.V, v);
    float above = 0.0f;
    int cnt = 0;
#pragma unroll
    for (int e = 0; e < kBlkElems<DT>; ++e) {
      above += above_w(v[e]);
      cnt += __popcll(__ballot(is_cand(v[e])));
    }
    above = wave_sum(above);
    __syncthreads();  // the previous chunk's wcnt / scratch / mbase are read
    if (l == 0) {
      sh.wcnt[w] = cnt;
      sh.scratch[w] = above;
    }
    __syncthreads();
    if (tid == 0) {
      int ct = 0;
      float ab = 0.0f;
      for (int q = 0; q < kSelWaves; ++q) {
        ct += sh.wcnt[q];
        ab += sh.scratch[q];
      }
      const int at = atomicAdd(&sh.ncand, ct);
      if (at + ct > kCandCap) sh.over = 1;
      sh.mbase = at;
      sh.ccnt[c] = ct;
      sh.cbeg[c] = at;
      sh.cabove[c] = ab;
    }
    __syncthreads();
    if (sh.mbase + sh.ccnt[c] <= kCandCap) {
      int pos = sh.mbase;
      for (int q = 0; q < w; ++q) pos += sh.wcnt[q];
#pragma unroll
      for (int e = 0; e < kBlkElems<DT>; ++e) put(v[e], pos);
    }
  }
  __syncthreads();
  src.n = sh.ncand;
  src.lds = sh.over == 0;
  // Weight above the range: every token there is kept.
  float base = 0.0f;
  for (int c = l; c < nc; c += kWave) base += sh.cabove[c];
  base = wave_sum(base);
  __syncthreads();
  const KeySpan ks = key_span(src, sh);
  unsigned kmin = 0;
  if (mode & 1) kmin = select_kth(src, sh, ks, krem);
  unsigned key = kmin;
  if (mode & 2) {
    // top-p's share is of what top-k kept: with top-k, base plus the
    // candidates at or above kmin (everything below the range is below the
    // k-th largest); without, the whole row.
    float zk = Z;
    if (mode & 1) {
      float zc = 0.0f;
      src.each([&](unsigned k2) {
        if (k2 >= kmin) zc += fast_exp2((fkey_inv(k2) - m) * kk);
      });
      zk = base + block_sum(zc, sh.scratch);
    }
    const float t = tp * zk - base;
    if (t > 0.0f) {
      key = select_mass(src, sh, ks, t, kmin, m, kk);
    } else {
      // The range is chosen so that this does not happen (the share above
      // it stays below top_p); keep the top candidate group if it does.
      if (tid == 0) sh.minkey = 0;
      __syncthreads();
      src.each([&](unsigned k2) { atomicMax(&sh.minkey, k2); });
      __syncthreads();
      key = sh.minkey;
    }
  }
  // Kept weight per chunk: above the range, plus its candidates at or above
  // the threshold (a wavefront per chunk, a fixed order).
  for (int c = w; c < nc; c += kSelWaves) {
    float kept = 0.0f;
    if (src.lds) {
      for (int f = sh.cbeg[c] + l; f < sh.cbeg[c] + sh.ccnt[c]; f += kWave) {
        const unsigned k2 = sh.key[f];
        if (k2 >= key) kept += fast_exp2((fkey_inv(k2) - m) * kk);
      }
    } else {
      src.chunk(c, [&](float v) {
        if (is_cand(v) && fkey(v) >= key) kept += fast_exp2((v - m) * kk);
      });
    }
    kept = wave_sum(kept) + sh.cabove[c];
    if (l == 0) {
      a.tpart[h0 + c] = kept;
      sh.ckept[c] = kept;
    }
  }
  __syncthreads();
  if (w == 0) {
    float tot = 0.0f;
    for (int c = l; c < nc; c += kWave) tot += sh.ckept[c];
    tot = wave_sum(tot);
    if (l == 0) a.tinfo[row] = f32x4{fkey_inv(key), tot, 1.0f, 0.0f};
  }
}

template <int DT, bool VP>
int launch_t(const Args& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.B * (a.K + 1);
  hipLaunchKernelGGL((trunc_select_kernel<DT, VP>), dim3((unsigned)rows),
                     dim3(kSelThreads), 0, s, a);
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
