// Verification of a draft tree ([P3] gogongxt notes "SGLang 的实现": the
// target-only tree sampling, with both of its acceptance thresholds at 1,
// which is its lossless case). Node 0 of a sequence's tree is the root (the
// last committed token); node i >= 1 carries a drafted token and a parent
// before it, and logit row i scores the token after the path root..i.
// Children are tried in node order: at depth t (t tokens accepted so far)
// each child adds its target probability to a running sum, and the first
// child whose sum reaches the depth's coin u[t] is accepted. When none does,
// the final token is drawn with u[N-1] from the target with every child's
// token taken out; at a leaf it is drawn from the leaf's row. At T = 0 the
// child carrying the row's argmax is accepted, else the argmax is emitted.
//
// Design for gfx950: the stream pass (stream.hip) reads every node's row once
// (the rows j <= n_nodes - 1 of the linear layout) and leaves its chunk
// partials. This kernel takes one workgroup per sequence: wavefront 0 holds
// node i in lane i (trees of at most 64 nodes), gathers each node's token
// logit from its parent's row (one load per lane, all at once), the four
// wavefronts combine the rows' partials (requested with the sequence's
// parameters and cached in LDS when they fit), and wavefront 0 walks the tree: the
// children of the current node are a ballot of parent == node, their running
// sum is one wavefront prefix sum in node order, the accepted child the first
// lane of a ballot. The final draw picks its chunk from the partials minus
// the children's weight per chunk and re-reads only that chunk (one quarter
// of it on the vector path: the stream pass's quarter sums, minus the
// children's terms in their quarters).
#include "draw.h"

namespace specsam {
namespace {

static_assert(SS_MAX_TREE <= kWave, "one lane per tree node");

// The children's tokens a rejection removes from the final draw.
struct TokenList {
  const int* list;
  int n;
  __device__ __forceinline__ bool operator()(int i) const {
    for (int k = 0; k < n; ++k)
      if (list[k] == i) return true;
    return false;
  }
};

// Chunk partials of all N rows are cached in LDS when they fit.
constexpr int kTreeCache = 1024;
constexpr int kTreePer = kTreeCache / kThreads;  // partials a thread requests

struct TreeShared {
  f32x4 pc[kTreeCache];
  f32x4 wc[kTreeCache];  // the chunks' quarter sums (SL)
  int tok[kWave];
  int par[kWave];
  float u[kWave];
  float m[kWave];
  float s[kWave];
  int idx[kWave];
  int bad[kWave];
  int ptok[kWave];  // emitted tokens and the nodes they came from
  int pnode[kWave];
  int excl[kWave];
  float exw[kWave];        // their weights in the final node's row
  float xsum[kMaxChunks];  // weight of the removed tokens, per chunk
  int st, depth, cur, nexcl, all_excluded;
  ChunkPick pick;
  DrawShared draw;
};

// SL: the final draw re-reads one quarter of its chunk (vector path, the
// partials and quarter sums of all N rows cached; the launch guarantees
// both).
template <int DT, bool VP, bool SL>
__global__ __launch_bounds__(kThreads) void spec_tree_finalize_kernel(
    Args a, const int32_t* tokens, const int32_t* parent, int32_t* out_nodes) {
  constexpr bool slices = VP && SL;
  __shared__ TreeShared sh;
  const int tid = threadIdx.x, w = tid / kWave, l = tid % kWave;
  const int b = blockIdx.x;
  const int N = a.K + 1, nc = a.nchunks;
  const int64_t row0 = (int64_t)b * N;
  // Everything that depends on no other load is requested at once: the
  // sequence's parameters, every node's token, parent and coin (lanes of
  // wavefront 0), and the chunk partials of all N rows when they fit the
  // LDS cache (kTreePer per thread, the index clamped rather than tested, so
  // that none of them waits for another). Rows and nodes past n_nodes are
  // read but not used.
  const bool cached = N * nc <= kTreeCache;  // uniform
  const f32x4* P0 = a.partials + row0 * nc;
  f32x4 pv[kTreePer], wv[kTreePer];
  if (cached) {
#pragma unroll
    for (int i = 0; i < kTreePer; ++i) {
      pv[i] = P0[min(tid + i * kThreads, N * nc - 1)];
      if constexpr (slices) wv[i] = a.wparts[row0 * nc + min(tid + i * kThreads, N * nc - 1)];
    }
  }
  int tk = 0, pr = -1;
  float uu = 0.0f;
  if (w == 0) {
    tk = tokens[row0 + min(l, N - 1)];
    pr = parent[row0 + min(l, N - 1)];
    if (l < N && a.uniforms) uu = a.uniforms[row0 + l];
  }
  int d;
  float T;
  const int st0 = seq_check(a, b, &d, &T);  // d = n_nodes - 1
  if (cached) {
#pragma unroll
    for (int i = 0; i < kTreePer; ++i)
      if (tid + i * kThreads < N * nc) {
        sh.pc[tid + i * kThreads] = pv[i];
        if constexpr (slices) sh.wc[tid + i * kThreads] = wv[i];
      }
  }
  if (st0) {
    if (tid == 0) atomicOr(&a.status[b], st0);
    return;
  }
  const int n = d + 1;
  const bool greedy = (T == 0.0f);
  const float kk = greedy ? 0.0f : kLog2e / T;
  // Nodes, one per lane of wavefront 0, and the tree's validity.
  if (w == 0) {
    if (l >= n) {
      tk = 0;
      pr = -1;
    }
    int bad = 0;
    if (l == 0) bad = pr != -1;
    else if (l < n) bad = pr < 0 || pr >= l || tk < 0 || tk >= a.V;
    sh.tok[l] = tk;
    sh.par[l] = pr;
    sh.u[l] = uu;
    bad = wave_or(bad);
    if (l == 0) sh.st = bad ? SS_ST_TREE : 0;
  }
  __syncthreads();
  if (w == 0 && sh.st == 0) {
    // siblings must carry distinct tokens
    int dup = 0;
    if (l >= 1 && l < n)
      for (int j = 1; j < l; ++j) dup |= (sh.par[j] == sh.par[l] && sh.tok[j] == sh.tok[l]);
    dup = wave_or(dup);
    if (l == 0 && dup) sh.st = SS_ST_TREE;
  }
  __syncthreads();
  if (sh.st) {
    if (tid == 0) atomicOr(&a.status[b], sh.st);
    return;
  }
  // Each node's token logit in its parent's row (T > 0 only), kept by its
  // lane until the walk (stored to LDS, it would be waited for at once).
  float lxr = 0.0f;
  if (w == 0 && !greedy && l >= 1 && l < n)
    lxr = load_one<DT>(a.logits + (row0 + sh.par[l]) * a.V * Dt<DT>::kBytes, sh.tok[l]);
  // Partial of chunk c of row j: from the cache, or from the workspace.
  auto part = [&](int j, int c) {
    return cached ? sh.pc[j * nc + c] : load_partial(P0 + (int64_t)j * nc + c);
  };
  // Row statistics from the chunk partials, one wavefront per row. (The two
  // sources are separate instantiations: a choice per access would make the
  // LDS reads wait for the loads in flight, the node logits among them.)
  auto combine_rows = [&](auto partf) {
    for (int j = w; j < n; j += kWaves) {
      if (greedy) {
        float bv = kNegInf, m1 = kNegInf, s1 = 0.0f;
        int bi = INT_MAX;
        for (int c = l; c < nc; c += kWave) {
          const f32x4 p = partf(j, c);
          argmax_merge(bv, bi, p.x, __float_as_int(p.w));
          lse_merge(m1, s1, p.x, p.y, kLog2e);
        }
        wave_argmax(bv, bi);
        wave_lse(m1, s1, kLog2e);
        if (l == 0) {
          sh.idx[j] = bi;
          sh.bad[j] = !(s1 > 0.0f) || !isfinite(s1) || bv == INFINITY || bv == kNegInf;
        }
      } else {
        float m = kNegInf, s = 0.0f;
        for (int c = l; c < nc; c += kWave) {
          const f32x4 p = partf(j, c);
          lse_merge(m, s, p.x, p.y, kk);
        }
        wave_lse(m, s, kk);
        if (l == 0) {
          sh.m[j] = m;
          sh.s[j] = s;
          sh.bad[j] = !(s > 0.0f) || !isfinite(s) || !isfinite(m);
        }
      }
    }
  };
  if (cached)
    combine_rows([&](int j, int c) { return sh.pc[j * nc + c]; });
  else
    combine_rows([&](int j, int c) { return load_partial(P0 + (int64_t)j * nc + c); });
  __syncthreads();
  // The walk (wavefront 0).
  if (w == 0) {
    int badrow = (l < n) ? sh.bad[l] : 0;
    badrow = wave_or(badrow);
    if (badrow) {
      if (l == 0) {
        atomicOr(&a.status[b], SS_ST_NONFINITE);
        sh.st = SS_ST_NONFINITE;
      }
    } else {
      const int mytok = (l < n) ? sh.tok[l] : -1;
      const int mypar = (l >= 1 && l < n) ? sh.par[l] : -2;
      const float mylx = (l >= 1 && l < n && !greedy) ? lxr : 0.0f;
      int cur = 0, depth = 0;
      while (true) {
        const bool child = (mypar == cur);
        int next = -1;
        if (greedy) {
          const unsigned long long hit = __ballot(child && mytok == sh.idx[cur]);
          if (hit) next = __ffsll((unsigned long long)hit) - 1;
        } else if (__ballot(child)) {
          const float p = child ? fast_exp2((mylx - sh.m[cur]) * kk) / sh.s[cur] : 0.0f;
          const float run = wave_inclusive_sum(p);
          const unsigned long long hit = __ballot(child && sh.u[depth] <= run);
          if (hit) next = __ffsll((unsigned long long)hit) - 1;
        }
        if (next < 0) break;
        if (l == 0) {
          sh.ptok[depth] = sh.tok[next];
          sh.pnode[depth] = next;
        }
        cur = next;
        ++depth;
      }
      // The children of the final node leave the final draw.
      const bool child = (mypar == cur);
      const unsigned long long cm = __ballot(child);
      if (child) {
        const int k = __popcll(cm & ((1ull << l) - 1));
        sh.excl[k] = mytok;
        // (with quarters: the token's term in its chunk's own frame, as the
        // stream pass formed it)
        const float ref =
            slices ? sh.pc[cur * nc + mytok / kChunk<DT>].x : sh.m[cur];
        sh.exw[k] = greedy ? 0.0f : fast_exp2((mylx - ref) * kk);
      }
      if (l == 0) {
        sh.cur = cur;
        sh.depth = depth;
        sh.nexcl = __popcll(cm);
        sh.st = 0;
      }
    }
  }
  for (int c = tid; c < nc; c += kThreads) sh.xsum[c] = 0.0f;
  __syncthreads();
  if (sh.st) return;
  const int cur = sh.cur, depth = sh.depth;
  int tok;
  if (greedy) {
    tok = sh.idx[cur];
  } else if constexpr (slices) {
    if (w == 0) {
      // Quarter weights of chunk c in row cur, the children's terms taken
      // out of their quarters in node order. A quarter that only the removed
      // tokens filled is left with a rounding residue of either sign when
      // several of them share it; a remainder within 2^-20 of what was
      // removed counts as nothing (a coin that only such a sliver would
      // separate is within 1e-6 of a breakpoint of the exact draw).
      const float m = sh.m[cur], uK = sh.u[N - 1];
      const int nx = sh.nexcl;
      auto quarters = [&](int c, bool excl) {
        const f32x4 qs = sh.wc[cur * nc + c];
        const double sc = chunk_scale(sh.pc[cur * nc + c].x, m, kk);
        double sq[4] = {qs.x, qs.y, qs.z, qs.w}, rm[4] = {0.0, 0.0, 0.0, 0.0};
        if (excl) {
          for (int k = 0; k < nx; ++k) {
            const int t = sh.excl[k];
            if (t / kChunk<DT> != c) continue;
            const int q = (t - c * kChunk<DT>) / kVec<DT> / kThreads / 2;
            const double x = sh.exw[k];
#pragma unroll
            for (int i = 0; i < 4; ++i)
              if (i == q) {
                sq[i] -= x;
                rm[i] += x;
              }
          }
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sq[i] = (rm[i] > 0.0 && sq[i] <= rm[i] * 0x1p-20) ? 0.0 : fmax(0.0, sq[i]);
        }
        return QuarterW{sq[0] * sc, sq[1] * sc, sq[2] * sc, sq[3] * sc};
      };
      ChunkPick pk = pick_chunk_slice(nc, uK, [&](int c) { return quarters(c, true); });
      int allx = 0;
      if (pk.chunk < 0) {
        // Rounding left nothing outside the children: draw from the row.
        pk = pick_chunk_slice(nc, uK, [&](int c) { return quarters(c, false); });
        allx = 1;
      }
      if (l == 0) {
        sh.pick = pk;
        sh.all_excluded = allx;
      }
    }
    __syncthreads();
    u32x4 rs[kSliceLoads];
    draw_load_slice<DT>(a, b, cur, sh.pick, rs);
    tok = draw_in_chunk<DT, VP, false, TokenList, NoDuring, NoQ, true>(
        a, sh.draw, b, cur, sh.pick, TokenList{sh.excl, sh.all_excluded ? 0 : sh.nexcl},
        sh.m[cur], kk, 0.0f, kNegInf, rs);
  } else {
    if (w == 0 && l < sh.nexcl) atomicAdd(&sh.xsum[sh.excl[l] / kChunk<DT>], sh.exw[l]);
    __syncthreads();
    if (w == 0) {
      const float m = sh.m[cur], uK = sh.u[N - 1];
      ChunkPick pk = pick_chunk(nc, uK, [&](int c) {
        const f32x4 p = part(cur, c);
        return fmax(0.0, chunk_weight(p.y, p.x, m, kk) - (double)sh.xsum[c]);
      });
      int allx = 0;
      if (pk.chunk < 0) {
        // Rounding left nothing outside the children: draw from the row.
        pk = pick_chunk(nc, uK, [&](int c) {
          const f32x4 p = part(cur, c);
          return chunk_weight(p.y, p.x, m, kk);
        });
        allx = 1;
      }
      if (l == 0) {
        sh.pick = pk;
        sh.all_excluded = allx;
      }
    }
    __syncthreads();
    u32x4 raw[kLoads];
    draw_load<DT, VP>(a, b, cur, sh.pick, raw);
    tok = draw_in_chunk<DT, VP, false>(
        a, sh.draw, b, cur, sh.pick, TokenList{sh.excl, sh.all_excluded ? 0 : sh.nexcl},
        sh.m[cur], kk, 0.0f, kNegInf, raw);
  }
  if (w == 0 && l < N) {
    int ot = -1, on = -1;
    if (l < depth) {
      ot = sh.ptok[l];
      on = sh.pnode[l];
    } else if (l == depth) {
      ot = tok;
      on = cur;
    }
    a.out[row0 + l] = ot;
    out_nodes[row0 + l] = on;
    if (l == 0) a.nem[b] = depth + 1;
  }
}

template <int DT, bool VP>
int launch_tree_t(const Args& a, const int32_t* tokens, const int32_t* parent,
                  int32_t* out_nodes, hipStream_t s) {
  const bool sl = VP && a.wparts != nullptr && (a.K + 1) * a.nchunks <= kTreeCache;
  if (sl)
    hipLaunchKernelGGL((spec_tree_finalize_kernel<DT, VP, true>), dim3((unsigned)a.B),
                       dim3(kThreads), 0, s, a, tokens, parent, out_nodes);
  else
    hipLaunchKernelGGL((spec_tree_finalize_kernel<DT, VP, false>), dim3((unsigned)a.B),
                       dim3(kThreads), 0, s, a, tokens, parent, out_nodes);
  return check_launch("spec_verify_tree");
}

}  // namespace

int launch_tree_finalize(const Args& a, bool f32, bool vp, const int32_t* tokens,
                         const int32_t* parent, int32_t* out_nodes, hipStream_t s) {
  return f32 ? (vp ? launch_tree_t<SS_DTYPE_F32, true>(a, tokens, parent, out_nodes, s)
                   : launch_tree_t<SS_DTYPE_F32, false>(a, tokens, parent, out_nodes, s))
             : (vp ? launch_tree_t<SS_DTYPE_BF16, true>(a, tokens, parent, out_nodes, s)
                   : launch_tree_t<SS_DTYPE_BF16, false>(a, tokens, parent, out_nodes, s));
}

}  // namespace specsam
