// Dynamic suffix automaton per sequence: extension and drafting.
//
// Method ([P1] cann-recipes-train article §1.1 "SAM 原理"; [P4] SAM-Decoding
// summary §3 "Suffix Automaton Construction", "Drafting with Suffix
// Automaton", "Update of Suffix Automaton"): states are endpos classes with
// len, link and min_endpos (first end position of the state's strings); every
// verified token extends the automaton by Blumer's online construction; the
// draft follows suffix links from the state of the whole text to the first
// state with an outgoing transition and copies the tokens that followed that
// state's first occurrence.
//
// Layout (one contiguous block per sequence, 256-byte aligned):
//   header  int32[16]: n, last, num_states, num_edges, status, max_len, V,
//           hash_slots, ...
//   states  int4[2*max_len]: (len, link, min_endpos, first_edge); one 16-byte
//           load brings every field a step of the construction reads.
//   text    int32[max_len]: committed tokens (the draft source).
//   hash    int4[hash_slots]: (src, token, dst, next) open-addressing table
//           keyed by (src, token), in 128-byte buckets of 8 rows probed
//           linearly; `next` chains a state's transitions so a clone can copy
//           them. hash_slots = next power of two >= 6*max_len keeps the load
//           at most 1/2 for the at most 3*max_len transitions.
//
// Execution: sam_extend runs one wavefront per sequence. The construction is a
// chain of dependent loads, so lanes do not split it; they cooperate on each
// hash probe (8 lanes read a whole bucket in one request, a ballot finds the
// key or the first empty row), and the next state record is loaded alongside
// each probe. Every lane performs the same stores with the same values, so
// each lane reads its own writes (no cross-lane ordering is assumed).
#include <algorithm>
#include <climits>

#include "internal.h"

namespace specsam {
namespace {

constexpr int kBucket = 8;  // rows per 128-byte bucket
constexpr int kMagic = 0x53414d31;

struct SamLayout {
  size_t states, text, slots, block;
  int hash_slots;
};

__host__ __device__ inline size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

__host__ __device__ inline SamLayout sam_layout(int max_len) {
  SamLayout L;
  size_t want = (size_t)6 * (size_t)max_len;
  size_t h = 64;
  while (h < want) h <<= 1;
  L.hash_slots = (int)h;
  L.states = 64;
  L.text = L.states + (size_t)2 * max_len * 16;
  L.slots = al256(L.text + (size_t)max_len * 4);
  L.block = al256(L.slots + h * 16);
  return L;
}

enum Hdr { H_N = 0, H_LAST, H_STATES, H_EDGES, H_STATUS, H_MAXLEN, H_V, H_SLOTS,
           H_MAGIC };

struct Seq {
  int* hdr;
  i32x4* st;
  int* text;
  i32x4* slots;
};

__device__ __forceinline__ Seq seq_at(unsigned char* base, int b, const SamLayout& L) {
  unsigned char* p = base + (size_t)b * L.block;
  return Seq{reinterpret_cast<int*>(p), reinterpret_cast<i32x4*>(p + L.states),
             reinterpret_cast<int*>(p + L.text),
             reinterpret_cast<i32x4*>(p + L.slots)};
}

__device__ __forceinline__ unsigned bucket_of(int s, int c, unsigned bmask) {
  unsigned long long k = ((unsigned long long)(unsigned)s << 32) | (unsigned)c;
  k ^= k >> 33;
  k *= 0xff51afd7ed558ccdull;
  k ^= k >> 33;
  k *= 0xc4ceb9fe1a85ec53ull;
  k ^= k >> 33;
  return (unsigned)k & bmask;
}

struct Probe {
  int slot;   // row of (s, c), or the first empty row in probe order; -1 if full
  bool found;
  int dst;
};

// Wave-cooperative lookup of (s, c). Uniform in, uniform out.
__device__ __forceinline__ Probe probe(const i32x4* slots, unsigned bmask, int s,
                                       int c) {
  const int l = lane_id();
  unsigned bk = bucket_of(s, c, bmask);
  for (unsigned it = 0; it <= bmask; ++it) {
    i32x4 v = i32x4{-2, -2, -2, -2};
    if (l < kBucket) v = slots[(size_t)bk * kBucket + l];
    const bool m = (l < kBucket) && v.x == s && v.y == c;
    const bool e = (l < kBucket) && v.x == -1;
    const unsigned long long bal = __ballot(m || e);
    if (bal) {
      const int f = __ffsll((unsigned long long)bal) - 1;
      Probe r;
      r.slot = (int)(bk * kBucket) + f;
      r.found = (__ballot(m) >> f) & 1ull;
      r.dst = __shfl(v.z, f, kWave);
      return r;
    }
    bk = (bk + 1) & bmask;
  }
  return Probe{-1, false, -1};
}

struct HdrRegs {
  int n, last, nstates, nedges, status, max_len, V, slots;
};

// Appends token c at position n (Blumer's online extension; `cur` is numbered
// before `clone`). Returns false if a bound check trips.
__device__ bool extend_one(const Seq& S, HdrRegs& h, int c, unsigned bmask) {
  const int i = h.n;
  const int cur = h.nstates++;
  i32x4 rp = S.st[h.last];
  S.st[cur] = i32x4{rp.x + 1, -1, i, -1};
  int p = h.last;
  Probe pr;
  int guard = 0;
  // Walk suffix links from last, adding (p, c) -> cur until (p, c) exists.
  while (true) {
    const int nxt = rp.y;
    i32x4 rn = i32x4{0, -1, -1, -1};
    if (nxt != -1) rn = S.st[nxt];  // in flight together with the probe
    pr = probe(S.slots, bmask, p, c);
    if (pr.slot < 0) return false;
    if (pr.found) break;
    S.slots[pr.slot] = i32x4{p, c, cur, rp.w};
    reinterpret_cast<int*>(&S.st[p])[3] = pr.slot;
    h.nedges++;
    p = nxt;
    if (p == -1) break;
    rp = rn;
    if (++guard > h.nstates) return false;
  }
  if (p == -1) {
    reinterpret_cast<int*>(&S.st[cur])[1] = 0;
  } else {
    const int q = pr.dst;
    const i32x4 rq = S.st[q];
    if (rp.x + 1 == rq.x) {
      reinterpret_cast<int*>(&S.st[cur])[1] = q;
    } else {
      const int clone = h.nstates++;
      // Copy q's transitions into the clone.
      int first = -1, e = rq.w, g2 = 0;
      while (e != -1) {
        const i32x4 se = S.slots[e];
        const Probe pc = probe(S.slots, bmask, clone, se.y);
        if (pc.slot < 0 || pc.found) return false;
        S.slots[pc.slot] = i32x4{clone, se.y, se.z, first};
        first = pc.slot;
        h.nedges++;
        e = se.w;
        if (++g2 > h.nedges) return false;
      }
      S.st[clone] = i32x4{rp.x + 1, rq.y, rq.z, first};
      // Redirect (p', c) -> q to the clone along the suffix path from p.
      int sl = pr.slot;
      i32x4 rr = rp;
      int g3 = 0;
      while (true) {
        reinterpret_cast<int*>(&S.slots[sl])[2] = clone;
        const int pp = rr.y;
        if (pp == -1) break;
        rr = S.st[pp];
        const Probe p3 = probe(S.slots, bmask, pp, c);
        if (p3.slot < 0 || !p3.found || p3.dst != q) break;
        sl = p3.slot;
        if (++g3 > h.nstates) return false;
      }
      reinterpret_cast<int*>(&S.st[q])[1] = clone;
      reinterpret_cast<int*>(&S.st[cur])[1] = clone;
    }
  }
  h.last = cur;
  S.text[i] = c;
  h.n = i + 1;
  return true;
}

__global__ __launch_bounds__(kWave) void sam_extend_kernel(
    unsigned char* base, int max_len, SamLayout L, const int32_t* tokens,
    int ld, const int32_t* counts) {
  const int b = blockIdx.x;
  const Seq S = seq_at(base, b, L);
  HdrRegs h;
  {
    const i32x4 h0 = reinterpret_cast<const i32x4*>(S.hdr)[0];
    const i32x4 h1 = reinterpret_cast<const i32x4*>(S.hdr)[1];
    h = HdrRegs{h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
  }
  if (h.status != 0) return;
  const unsigned bmask = (unsigned)(h.slots / kBucket) - 1u;
  const int cnt = counts[b];
  int st = 0;
  if (cnt < 0 || cnt > ld) {
    st = SS_ST_COUNT;
  } else {
    const int32_t* tk = tokens + (int64_t)b * ld;
    for (int t = 0; t < cnt; ++t) {
      const int c = tk[t];
      if (c < 0 || c >= h.V) {
        st = SS_ST_TOKEN_RANGE;
        break;
      }
      if (h.n >= max_len || h.nstates + 2 > 2 * max_len) {
        st = SS_ST_SAM_CAPACITY;
        break;
      }
      if (!extend_one(S, h, c, bmask)) {
        st = SS_ST_SAM_CAPACITY;
        break;
      }
    }
  }
  h.status |= st;
  reinterpret_cast<i32x4*>(S.hdr)[0] = i32x4{h.n, h.last, h.nstates, h.nedges};
  S.hdr[H_STATUS] = h.status;
}

// One lane per sequence: link walk, then a gather of up to K tokens.
__global__ __launch_bounds__(256) void sam_draft_kernel(
    const unsigned char* base, int B, SamLayout L, int K, int32_t* draft,
    int32_t* draft_len, int32_t* match_len) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const Seq S = seq_at(const_cast<unsigned char*>(base), b, L);
  const i32x4 h0 = reinterpret_cast<const i32x4*>(S.hdr)[0];
  const int n = h0.x, nstates = h0.z;
  int s = h0.y;
  i32x4 rs = S.st[s];
  for (int g = 0; s > 0 && rs.w == -1 && g < nstates; ++g) {
    s = rs.y;
    rs = S.st[s < 0 ? 0 : s];
  }
  const int Lm = (s < 0) ? 0 : rs.x;
  const int p = rs.z;
  const int d = (Lm == 0) ? 0 : min(K, n - 1 - p);
  for (int j = 0; j < K; ++j)
    draft[(int64_t)b * K + j] = (j < d) ? S.text[p + 1 + j] : -1;
  draft_len[b] = d;
  match_len[b] = Lm;
}

__global__ void sam_init_kernel(unsigned char* base, int max_len, int V,
                                SamLayout L) {
  const int b = blockIdx.y;
  const Seq S = seq_at(base, b, L);
  const size_t n = (size_t)L.hash_slots;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    S.slots[i] = i32x4{-1, -1, -1, -1};
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    reinterpret_cast<i32x4*>(S.hdr)[0] = i32x4{0, 0, 1, 0};
    reinterpret_cast<i32x4*>(S.hdr)[1] = i32x4{0, max_len, V, L.hash_slots};
    reinterpret_cast<i32x4*>(S.hdr)[2] = i32x4{kMagic, 0, 0, 0};
    reinterpret_cast<i32x4*>(S.hdr)[3] = i32x4{0, 0, 0, 0};
    S.st[0] = i32x4{0, -1, -1, -1};
  }
}

__global__ void sam_status_kernel(const unsigned char* base, int B, SamLayout L,
                                  int32_t* out) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const Seq S = seq_at(const_cast<unsigned char*>(base), b, L);
  out[b] = S.hdr[H_STATUS];
}

int check_dims(const char* fn, const void* state, int B, int max_len) {
  if (!state) return set_error(SS_EINVAL, "%s: state is NULL", fn);
  if ((uintptr_t)state & 255)
    return set_error(SS_EINVAL, "%s: state must be 256-byte aligned", fn);
  if (B < 1 || max_len < 1 || max_len > SS_MAX_LEN)
    return set_error(SS_EINVAL, "%s: need B >= 1 and 1 <= max_len <= %d", fn,
                     SS_MAX_LEN);
  return SS_OK;
}

}  // namespace
}  // namespace specsam

using namespace specsam;

extern "C" size_t sam_state_bytes(int B, int max_len) {
  if (B < 1 || max_len < 1 || max_len > SS_MAX_LEN) return 0;
  return (size_t)B * sam_layout(max_len).block;
}

extern "C" int sam_hash_slots(int max_len) {
  if (max_len < 1 || max_len > SS_MAX_LEN) return 0;
  return sam_layout(max_len).hash_slots;
}

extern "C" int sam_init(void* state, int B, int max_len, int V, void* stream) {
  int rc = check_dims("sam_init", state, B, max_len);
  if (rc) return rc;
  if (V < 1) return set_error(SS_EINVAL, "sam_init: V must be >= 1");
  if (B > 65535) return set_error(SS_EINVAL, "sam_init: B must be <= 65535");
  const SamLayout L = sam_layout(max_len);
  const unsigned gx = (unsigned)std::min<size_t>(
      ((size_t)L.hash_slots + 255) / 256, 1024);
  hipLaunchKernelGGL(sam_init_kernel, dim3(gx, (unsigned)B), dim3(256), 0,
                     as_stream(stream), reinterpret_cast<unsigned char*>(state),
                     max_len, V, L);
  return check_launch("sam_init");
}

extern "C" int sam_extend(void* state, int B, int max_len, const int32_t* tokens,
                          int ld_tokens, const int32_t* counts, void* stream) {
  int rc = check_dims("sam_extend", state, B, max_len);
  if (rc) return rc;
  if (!tokens || !counts || ld_tokens < 0)
    return set_error(SS_EINVAL, "sam_extend: tokens/counts NULL or ld < 0");
  const SamLayout L = sam_layout(max_len);
  hipLaunchKernelGGL(sam_extend_kernel, dim3((unsigned)B), dim3(kWave), 0,
                     as_stream(stream), reinterpret_cast<unsigned char*>(state),
                     max_len, L, tokens, ld_tokens, counts);
  return check_launch("sam_extend");
}

extern "C" int sam_draft(const void* state, int B, int max_len, int K,
                         int32_t* draft, int32_t* draft_len, int32_t* match_len,
                         void* stream) {
  int rc = check_dims("sam_draft", state, B, max_len);
  if (rc) return rc;
  if (K < 1 || K > SS_MAX_K)
    return set_error(SS_EINVAL, "sam_draft: need 1 <= K <= %d", SS_MAX_K);
  if (!draft || !draft_len || !match_len)
    return set_error(SS_EINVAL, "sam_draft: output pointer is NULL");
  const SamLayout L = sam_layout(max_len);
  hipLaunchKernelGGL(sam_draft_kernel, dim3((unsigned)((B + 255) / 256)),
                     dim3(256), 0, as_stream(stream),
                     reinterpret_cast<const unsigned char*>(state), B, L, K,
                     draft, draft_len, match_len);
  return check_launch("sam_draft");
}

extern "C" int sam_status(const void* state, int B, int max_len,
                          int32_t* status_out, void* stream) {
  int rc = check_dims("sam_status", state, B, max_len);
  if (rc) return rc;
  if (!status_out) return set_error(SS_EINVAL, "sam_status: status_out is NULL");
  const SamLayout L = sam_layout(max_len);
  hipLaunchKernelGGL(sam_status_kernel, dim3((unsigned)((B + 255) / 256)),
                     dim3(256), 0, as_stream(stream),
                     reinterpret_cast<const unsigned char*>(state), B, L,
                     status_out);
  return check_launch("sam_status");
}

extern "C" int sam_export(const void* state, int B, int max_len, int b,
                          int32_t* header_out, int32_t* states_out,
                          int32_t* edges_out, int32_t* text_out, void* stream) {
  int rc = check_dims("sam_export", state, B, max_len);
  if (rc) return rc;
  if (b < 0 || b >= B) return set_error(SS_EINVAL, "sam_export: b out of range");
  const SamLayout L = sam_layout(max_len);
  const unsigned char* p =
      reinterpret_cast<const unsigned char*>(state) + (size_t)b * L.block;
  hipStream_t s = as_stream(stream);
  struct Part {
    void* dst;
    size_t off, bytes;
  } parts[4] = {{header_out, 0, 8 * sizeof(int32_t)},
                {states_out, L.states, (size_t)2 * max_len * 16},
                {edges_out, L.slots, (size_t)L.hash_slots * 16},
                {text_out, L.text, (size_t)max_len * 4}};
  for (const Part& pt : parts) {
    if (!pt.dst) continue;
    hipError_t e = hipMemcpyAsync(pt.dst, p + pt.off, pt.bytes,
                                  hipMemcpyDeviceToDevice, s);
    if (e != hipSuccess)
      return set_error(SS_ELAUNCH, "sam_export: %s", hipGetErrorString(e));
  }
  return SS_OK;
}
