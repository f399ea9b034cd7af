// Stand-alone suffix-automaton kernels: init, extend, draft, status.
//
// The device code (layout, Blumer extension, drafting) is in sam_device.h and
// follows [P1] cann-recipes-train article §1.1 "SAM 原理" and [P4] SAM-Decoding
// summary §3; the fused step kernel in verify.hip runs the same functions.
#include <algorithm>
#include <climits>

#include "sam_device.h"

namespace specsam {
namespace {

// One wavefront per sequence.
__global__ __launch_bounds__(kWave) void sam_extend_kernel(
    unsigned char* base, int max_len, SamLayout L, const int32_t* tokens,
    int ld, const int32_t* counts) {
  const int b = blockIdx.x;
  const SamSeq S = sam_seq(base, b, L);
  SamCursor cs = sam_open(S);
  sam_append(S, cs, tokens + (int64_t)b * ld, counts[b], ld, max_len);
}

// The same extension with work counters, summed into stats[SS_STAT_COUNT].
__global__ __launch_bounds__(kWave) void sam_extend_stats_kernel(
    unsigned char* base, int max_len, SamLayout L, const int32_t* tokens,
    int ld, const int32_t* counts, unsigned long long* stats) {
  const int b = blockIdx.x;
  SamCounters ctr = {};
  const SamSeq S = sam_seq(base, b, L);
  SamCursor cs = sam_open(S);
  sam_append<true>(S, cs, tokens + (int64_t)b * ld, counts[b], ld, max_len, &ctr);
  if (lane_id() < SS_STAT_COUNT) {
    unsigned long long v = 0;
#pragma unroll
    for (int k = 0; k < SS_STAT_COUNT; ++k)
      if (lane_id() == k) v = ctr.v[k];
    atomicAdd(stats + lane_id(), v);
  }
}

// One wavefront per sequence.
__global__ __launch_bounds__(kWave) void sam_draft_kernel(
    const unsigned char* base, SamLayout L, int K, int32_t* draft,
    int32_t* draft_len, int32_t* match_len) {
  const int b = blockIdx.x;
  sam_draft_seq(sam_seq(const_cast<unsigned char*>(base), b, L), K,
                draft + (int64_t)b * K, draft_len + b, match_len + b);
}

// Draft tree of up to M candidates (one wavefront per sequence; lane v holds
// tree node v): the state the single draft's link walk reaches, then its
// suffix-link ancestors, each giving the tokens after its first occurrence
// (K at most, cut at the end of the text). Each candidate is inserted into
// the trie token by token: a ballot over the nodes finds the child of the
// current node with that token, or the next free lane becomes one. Node 0 is
// the root; children keep their candidates' order.
__global__ __launch_bounds__(kWave) void sam_draft_tree_kernel(
    const unsigned char* base, SamLayout L, int K, int M, int N, int32_t* tok_out,
    int32_t* par_out, int32_t* n_out, int32_t* mlen_out) {
  const int b = blockIdx.x;
  const int l = lane_id();
  const SamSeq S = sam_seq(const_cast<unsigned char*>(base), b, L);
  const SamCursor cs = sam_open(S);
  const int n = cs.h.n, nstates = cs.h.nstates;
  int s = cs.h.last;
  i32x4 rs = cs.rlast;
  for (int g = 0; s > 0 && rs.w == -1 && g < nstates; ++g) {
    s = rs.y;
    rs = S.st[s < 0 ? 0 : s];
  }
  const int ml = (s <= 0) ? 0 : rs.x;
  int ntok = -1, npar = -1;  // this lane's node
  int nn = 1;
  for (int i = 0; i < M && s > 0 && rs.x > 0; ++i) {
    const int p = rs.z;
    const int d = min(K, n - 1 - p);
    const int tv = (l < d) ? S.text[p + 1 + l] : -1;
    int cur = 0;
    for (int j = 0; j < d; ++j) {
      const int t = __builtin_amdgcn_readlane(tv, j);
      const unsigned long long hit =
          __ballot(l >= 1 && l < nn && npar == cur && ntok == t);
      if (hit) {
        cur = __ffsll((unsigned long long)hit) - 1;
      } else {
        if (l == nn) {
          npar = cur;
          ntok = t;
        }
        cur = nn++;
      }
    }
    s = rs.y;
    rs = S.st[s < 0 ? 0 : s];
  }
  if (l < N) {
    tok_out[(int64_t)b * N + l] = (l < nn) ? ntok : -1;
    par_out[(int64_t)b * N + l] = (l < nn) ? npar : -1;
  }
  if (l == 0) {
    n_out[b] = nn;
    if (mlen_out) mlen_out[b] = ml;
  }
}

// Extend then draft in one pass (the per-step pair, one launch).
__global__ __launch_bounds__(kWave) void sam_extend_draft_kernel(
    unsigned char* base, int max_len, SamLayout L, const int32_t* tokens,
    int ld, const int32_t* counts, int K, int32_t* draft, int32_t* draft_len,
    int32_t* match_len) {
  const int b = blockIdx.x;
  const SamSeq S = sam_seq(base, b, L);
  SamCursor cs = sam_open(S);
  if (sam_append(S, cs, tokens + (int64_t)b * ld, counts[b], ld, max_len))
    sam_draft_cursor(S, cs, K, draft + (int64_t)b * K, draft_len + b, match_len + b);
  else
    sam_draft_seq(S, K, draft + (int64_t)b * K, draft_len + b, match_len + b);
}

// Static automaton matching ([P4] SAM-Decoding summary §3, "Drafting with
// Suffix Automaton", "Update of Suffix Automaton"): match[b] = (state, length)
// of the longest suffix of sequence b's text that occurs in the static
// automaton's reference text. Each token t: take the state's transition on t
// if it has one (the match grows by one), else follow suffix links to the
// first state that has one (the match becomes that state's longest string
// plus t), or end at the root with an empty match. The state's record is
// requested together with each probe. Then, when K > 0, the static draft is
// the K tokens after the state's min_endpos (cut at the end of the text,
// none for an empty match), and with dynamic drafts given the static one is
// taken only when its match is longer by more than delta. One wavefront per
// sequence; the static automaton is read only.
__global__ __launch_bounds__(kWave) void sam_match_kernel(
    const unsigned char* sbase, SamLayout L, int32_t* match, const int32_t* tokens,
    int ld, const int32_t* counts, int K, int delta, const int32_t* dyn_draft,
    const int32_t* dyn_len, const int32_t* dyn_match, int32_t* draft,
    int32_t* draft_len, int32_t* source, int32_t* status) {
  const int b = blockIdx.x;
  const int l = lane_id();
  const SamSeq S = sam_seq(const_cast<unsigned char*>(sbase), 0, L);
  const i32x4 h0 = reinterpret_cast<const i32x4*>(S.hdr)[0];
  const i32x4 h1 = reinterpret_cast<const i32x4*>(S.hdr)[1];
  const int n = h0.x;
  const unsigned bmask = (unsigned)(h1.w / kBucket) - 1u;
  int s = match[2 * b], m = match[2 * b + 1];
  if (s < 0 || s >= h0.z || m < 0) {  // not a state of this automaton: the root
    s = 0;
    m = 0;
  }
  // A match longer than the state's longest string is not a match state of
  // this automaton either.
  if (m > S.st[s].x) {
    s = 0;
    m = 0;
  }
  int cnt = counts ? counts[b] : 0;
  if (cnt < 0 || cnt > ld) {  // reported; no token is read
    if (l == 0 && status) atomicOr(status + b, SS_ST_COUNT);
    cnt = 0;
  }
  for (int i = 0; i < cnt; ++i) {
    const int t = tokens[(int64_t)b * ld + i];
    bool take_len = false;
    while (true) {
      const i32x4 rc = S.st[s];  // in flight with the probe
      const SamProbe pr = sam_probe(S.slots, bmask, s, t);
      if (take_len) m = rc.x;
      if (pr.found) {
        s = pr.dst;
        m += 1;
        break;
      }
      if (s == 0) {
        m = 0;
        break;
      }
      s = rc.y;
      take_len = true;
    }
  }
  if (l == 0) {
    match[2 * b] = s;
    match[2 * b + 1] = m;
  }
  if (K <= 0) return;
  const i32x4 rs = S.st[s];
  const int d = (m == 0) ? 0 : min(K, n - 1 - rs.z);
  bool use = true;
  if (dyn_draft) use = m > dyn_match[b] + delta;
  if (l < K) {
    int v;
    if (use)
      v = (l < d) ? S.text[rs.z + 1 + l] : -1;
    else
      v = dyn_draft[(int64_t)b * K + l];
    draft[(int64_t)b * K + l] = v;
  }
  if (l == 0) {
    draft_len[b] = use ? d : dyn_len[b];
    if (source) source[b] = use ? 1 : 0;
  }
}

__global__ void sam_init_kernel(unsigned char* base, int max_len, int V,
                                SamLayout L) {
  const int b = blockIdx.y;
  const SamSeq S = sam_seq(base, b, L);
  const size_t n = (size_t)L.hash_slots;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (size_t)gridDim.x * blockDim.x)
    S.slots[i] = i32x4{-1, -1, -1, -1};
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    reinterpret_cast<i32x4*>(S.hdr)[0] = i32x4{0, 0, 1, 0};
    reinterpret_cast<i32x4*>(S.hdr)[1] = i32x4{0, max_len, V, L.hash_slots};
    reinterpret_cast<i32x4*>(S.hdr)[2] = i32x4{kSamMagic, 0, 0, 0};
    reinterpret_cast<i32x4*>(S.hdr)[3] = i32x4{0, 0, 0, 0};
    S.st[0] = i32x4{0, -1, -1, -1};
  }
}

__global__ void sam_status_kernel(const unsigned char* base, int B, SamLayout L,
                                  int32_t* out) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= B) return;
  const SamSeq S = sam_seq(const_cast<unsigned char*>(base), b, L);
  out[b] = S.hdr[H_STATUS];
}

constexpr bool kSamMatchSwitchedOff = true;

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

extern "C" int sam_extend_stats(void* state, int B, int max_len,
                                const int32_t* tokens, int ld_tokens,
                                const int32_t* counts, unsigned long long* stats,
                                void* stream) {
  int rc = check_dims("sam_extend_stats", state, B, max_len);
  if (rc) return rc;
  if (!tokens || !counts || ld_tokens < 0 || !stats)
    return set_error(SS_EINVAL, "sam_extend_stats: null pointer or ld < 0");
  const SamLayout L = sam_layout(max_len);
  hipLaunchKernelGGL(sam_extend_stats_kernel, dim3((unsigned)B), dim3(kWave), 0,
                     as_stream(stream), reinterpret_cast<unsigned char*>(state),
                     max_len, L, tokens, ld_tokens, counts, stats);
  return check_launch("sam_extend_stats");
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
  hipLaunchKernelGGL(sam_draft_kernel, dim3((unsigned)B), dim3(kWave), 0,
                     as_stream(stream),
                     reinterpret_cast<const unsigned char*>(state), L, K, draft,
                     draft_len, match_len);
  return check_launch("sam_draft");
}

extern "C" int sam_draft_tree(const void* state, int B, int max_len, int K, int M,
                              int N, int32_t* tokens, int32_t* parent,
                              int32_t* n_nodes, int32_t* match_len, void* stream) {
  int rc = check_dims("sam_draft_tree", state, B, max_len);
  if (rc) return rc;
  if (K < 1 || M < 0 || (int64_t)M * K + 1 > N || N > SS_MAX_TREE)
    return set_error(SS_EINVAL, "sam_draft_tree: need K >= 1, M >= 0 and "
                                "1 + M*K <= N <= %d (got K=%d M=%d N=%d)",
                     SS_MAX_TREE, K, M, N);
  if (!tokens || !parent || !n_nodes)
    return set_error(SS_EINVAL, "sam_draft_tree: output pointer is NULL");
  const SamLayout L = sam_layout(max_len);
  hipLaunchKernelGGL(sam_draft_tree_kernel, dim3((unsigned)B), dim3(kWave), 0,
                     as_stream(stream), reinterpret_cast<const unsigned char*>(state),
                     L, K, M, N, tokens, parent, n_nodes, match_len);
  return check_launch("sam_draft_tree");
}

extern "C" int sam_extend_draft(void* state, int B, int max_len,
                                const int32_t* tokens, int ld_tokens,
                                const int32_t* counts, int K, int32_t* draft,
                                int32_t* draft_len, int32_t* match_len,
                                void* stream) {
  int rc = check_dims("sam_extend_draft", state, B, max_len);
  if (rc) return rc;
  if (!tokens || !counts || ld_tokens < 0)
    return set_error(SS_EINVAL, "sam_extend_draft: tokens/counts NULL or ld < 0");
  if (K < 1 || K > SS_MAX_K)
    return set_error(SS_EINVAL, "sam_extend_draft: need 1 <= K <= %d", SS_MAX_K);
  if (!draft || !draft_len || !match_len)
    return set_error(SS_EINVAL, "sam_extend_draft: output pointer is NULL");
  const SamLayout L = sam_layout(max_len);
  hipLaunchKernelGGL(sam_extend_draft_kernel, dim3((unsigned)B), dim3(kWave), 0,
                     as_stream(stream), reinterpret_cast<unsigned char*>(state),
                     max_len, L, tokens, ld_tokens, counts, K, draft, draft_len,
                     match_len);
  return check_launch("sam_extend_draft");
}

extern "C" int sam_match(const void* static_state, int static_max_len, int B,
                         int32_t* match, const int32_t* tokens, int ld_tokens,
                         const int32_t* counts, int K, int delta,
                         const int32_t* dyn_draft, const int32_t* dyn_len,
                         const int32_t* dyn_match, int32_t* draft,
                         int32_t* draft_len, int32_t* source, int32_t* status,
                         void* stream) {
  // Switched off: one GPU run of this entry point's tests ended in a memory
  // fault, and the cause has not been shown (a bounds-checked host model of
  // the automaton kernels over the same inputs stays in bounds, and the
  // kernel's gfx950 code on the faulting call's path reads only in bounds).
  // The kernel stays in the source; the entry point refuses to launch it.
  if (kSamMatchSwitchedOff)
    return set_error(SS_EINVAL, "sam_match: switched off until the cause of a "
                                "GPU memory fault in its tests is shown");
  int rc = check_dims("sam_match", static_state, 1, static_max_len);
  if (rc) return rc;
  if (B < 1 || !match)
    return set_error(SS_EINVAL, "sam_match: need B >= 1 and a match array");
  if (counts && (!tokens || ld_tokens < 0))
    return set_error(SS_EINVAL, "sam_match: tokens NULL or ld < 0");
  if (K < 0 || K > SS_MAX_K)
    return set_error(SS_EINVAL, "sam_match: need 0 <= K <= %d", SS_MAX_K);
  if (K > 0 && (!draft || !draft_len))
    return set_error(SS_EINVAL, "sam_match: draft outputs are NULL");
  const int ndyn = (dyn_draft != nullptr) + (dyn_len != nullptr) + (dyn_match != nullptr);
  if (ndyn != 0 && ndyn != 3)
    return set_error(SS_EINVAL, "sam_match: give all dynamic-draft inputs or none");
  if (delta < 0) return set_error(SS_EINVAL, "sam_match: delta must be >= 0");
  const SamLayout L = sam_layout(static_max_len);
  hipLaunchKernelGGL(sam_match_kernel, dim3((unsigned)B), dim3(kWave), 0,
                     as_stream(stream),
                     reinterpret_cast<const unsigned char*>(static_state), L, match,
                     tokens, ld_tokens, counts, K, delta, dyn_draft, dyn_len,
                     dyn_match, draft, draft_len, source, status);
  return check_launch("sam_match");
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
