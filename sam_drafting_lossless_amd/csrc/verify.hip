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
// Design for gfx950: two kernels per step (two more when draft
// probabilities q are given), ordered by the stream they are launched on.
//   stream    (stream.hip) reads each needed logit row once and leaves one
//             partial per (row, 32 KiB chunk) in the workspace.
//   finalize  one workgroup per sequence: combines the chunk partials of each
//             row, judges the drafts with one wavefront (lane j judges draft
//             j; a ballot finds the first rejection), writes the outputs and,
//             for one-hot drafts or the bonus, draws the token (the chunk,
//             then one quarter of it, is picked from the rescaled quarter
//             sums and only that quarter is re-read; the whole chunk under
//             truncation). In the fused step it then extends the sequence's
//             automaton with the emitted tokens and writes the next draft.
//   residual  only when q is given: chunk sums of max(0, p - q) over the
//             rejected row, per quarter (sequence x chunk), then one
//             workgroup per sequence draws from them, re-reading a quarter.
// A design that let the last workgroup of each sequence finalize inside the
// stream kernel (agent-scope atomic hand-off) was measured slower: the
// finalize code raises the stream kernel's register count and its latency
// lands in the kernel's tail. For small launches too: with the partials
// stored at device scope, a ticket per streaming workgroup and one acquire
// in the last, a step took 22.8 us against 21.6 for the two kernels
// (B = 32, V = 151936, bf16, K = 5) and 14.9 against 14.6 (B = 1, V = 32):
// the hand-off's write-through, returning atomic and invalidate cost what
// the kernel boundary does. (A whole-cache fence in every workgroup took
// 89 us.)
#include <algorithm>
#include <atomic>
#include <mutex>

#include "draw.h"

namespace specsam {
namespace {

// Chunk partials of all K+1 rows are cached in LDS when they fit.
constexpr int kPartialCache = 1024;

struct FinalShared {
  f32x4 pc[kPartialCache];
  f32x4 wc[kPartialCache];  // the chunks' quarter sums (cached with pc)
  float m[kMaxRows];
  float s[kMaxRows];         // sum of the weights the row's decisions use
  float su[kMaxRows];        // untruncated sum (log-probabilities)
  float lam[kMaxRows];       // truncation threshold (-inf: none)
  float lx[kMaxRows];
  float u[kMaxRows];
  int idx[kMaxRows];
  int bad[kMaxRows];
  int x[kMaxRows];
  int tok[kMaxRows];
  float qx[kMaxRows];        // q at the draft token of each row
  ChunkPick pick[kMaxRows];  // chunk choice of a draw at each row (T > 0)
  int acc_len;
  int st;
  int hdr[8];  // the automaton's header, one dword per lane of wavefront 0
  int rec[4];  // the record of its last state
  DrawShared draw;
};

// Q: draft probabilities q are given (then SAM is false). SL: draws re-read
// one quarter of the chosen chunk (vector path, no truncation, partials
// cached: the launch guarantees all three).
template <int DT, bool VP, bool SAM, bool Q, bool SL>
__global__ __launch_bounds__(kThreads) void spec_finalize_kernel(Args a) {
  __shared__ FinalShared sh;
  const int tid = threadIdx.x, w = tid / kWave, l = tid % kWave;
  const int b = blockIdx.x;
  const int R = a.K + 1, nc = a.nchunks;
  // Everything that does not depend on another load is requested at once:
  // the sequence's parameters, drafts, coins, the partials of every row and
  // the automaton's header. The last wavefront then requests the record of
  // the automaton's last state and leaves both in LDS for the step
  // (wavefront 0) at the accept scan's barrier: the step's first loads then
  // wait for nothing but themselves and the draw's loads, requested just
  // before (load counters are in order: a record still in flight in
  // registers would make them wait for the draw's loads, and then take their
  // own round trip).
  int d;
  float T;
  const int st0 = seq_check(a, b, &d, &T);
  SamSeq S;
  SamCursor cs;
  if constexpr (SAM) S = sam_seq(a.sam, b, a.sl);
  const bool cached = R * nc <= kPartialCache;
  const f32x4* Pb = a.partials + (int64_t)b * R * nc;
  // All loads are issued before the first LDS store, so that they share one
  // round trip.
  // (The common case has at most one partial per thread; more go through a
  // plain loop.)
  const bool one = cached && R * nc <= kThreads;  // uniform
  // Quarter sums (the draw's slices); a row that was not streamed, or a
  // greedy one, leaves stale values no draw reads.
  constexpr bool slices = VP && SL;
  const f32x4* Wb = slices ? a.wparts + (int64_t)b * R * nc : nullptr;
  f32x4 pv = f32x4{0.0f, 0.0f, 0.0f, 0.0f}, wv = pv;
  if (one) {
    const int e = min(tid, R * nc - 1);
    pv = Pb[e];
    if constexpr (slices) wv = Wb[e];
  } else if (cached) {
    for (int e = tid; e < R * nc; e += kThreads) {
      sh.pc[e] = Pb[e];
      if constexpr (slices) sh.wc[e] = Wb[e];
    }
  }
  int xv = -1;
  float uv = 0.0f;
  if (tid < a.K) xv = a.draft[(int64_t)b * a.K + tid];
  if (tid < R && a.uniforms) uv = a.uniforms[(int64_t)b * R + tid];
  constexpr int kSamWave = kWaves - 1;
  int hv = 0, rv = 0;
  if constexpr (SAM) {
    if (w == kSamWave && l < 8) hv = S.hdr[l];
  }
  if (one && tid < R * nc) {
    sh.pc[tid] = pv;
    if constexpr (slices) sh.wc[tid] = wv;
  }
  if (tid < a.K) sh.x[tid] = xv;
  if (tid < R) sh.u[tid] = uv;
  __syncthreads();
  if (st0) {
    // Reported once; the automaton (if any) is left unchanged and the next
    // draft is taken from it as it is.
    if (tid == 0) {
      atomicOr(&a.status[b], st0);
      a.seqinfo[b] = i32x4{0, 0, 0, 0};
    }
    if constexpr (SAM) {
      if (w == 0)
        sam_draft_seq(sam_seq(a.sam, b, a.sl), a.K, a.next_draft + (int64_t)b * a.K,
                      a.next_draft_len + b, a.next_match_len + b);
    }
    return;
  }
  if constexpr (SAM) {
    if (w == kSamWave && l < 4)
      rv = reinterpret_cast<const int*>(S.st)[__builtin_amdgcn_readlane(hv, H_LAST) * 4 + l];
  }
  const bool greedy = (T == 0.0f);
  const float kk = greedy ? 0.0f : kLog2e / T;
  // Truncated target (top-k / top-p): the truncation passes left each row's
  // threshold and its kept probability per chunk.
  const bool trunc = a.tinfo != nullptr && trunc_active(a, b, T);
  // q at each draft token (1 for one-hot drafts), gathered while the rows
  // are combined so that the accept scan reads only LDS.
  if constexpr (Q) {
    if (!greedy && tid < d) {
      const int x = sh.x[tid];
      sh.qx[tid] = (x >= 0 && x < a.V) ? a.q[((int64_t)b * a.K + tid) * a.V + x] : 1.0f;
    }
  }
  // Row j's partials come from LDS when cached, else from the workspace. The
  // two sources are separate instantiations, so that LDS reads never wait
  // for global loads still in flight (a generic pointer, or a per-access
  // choice, would make them).
  auto combine_rows = [&](auto part) {
    for (int j = w; j <= d; j += kWaves) {
      if (greedy) {
        // argmax, and the sum of exp(l - max) at temperature 1 (NaN if the
        // row holds NaN)
        float bv = kNegInf, m1 = kNegInf, s1 = 0.0f;
        int bi = INT_MAX;
        for (int c = l; c < nc; c += kWave) {
          const f32x4 p = part(j, c);
          argmax_merge(bv, bi, p.x, __float_as_int(p.w));
          lse_merge(m1, s1, p.x, p.y, kLog2e);
        }
        wave_argmax(bv, bi);
        wave_lse(m1, s1, kLog2e);
        if (l == 0) {
          sh.m[j] = bv;
          sh.s[j] = s1;
          sh.idx[j] = bi;
          sh.bad[j] = !(s1 > 0.0f) || !isfinite(s1) || bv == INFINITY ||
                      bv == kNegInf;
        }
      } else {
        const int xj = (j < d) ? sh.x[j] : -1;
        const int cx = (xj >= 0 && xj < a.V) ? xj / kChunk<DT> : -1;
        float m = kNegInf, s = 0.0f, lxv = 0.0f;
        bool has = false;
        for (int c = l; c < nc; c += kWave) {
          const f32x4 p = part(j, c);
          lse_merge(m, s, p.x, p.y, kk);
          if (c == cx) {
            lxv = p.z;
            has = true;
          }
        }
        wave_lse(m, s, kk);
        const unsigned long long hb = __ballot(has);
        if (hb) lxv = readlane_f(lxv, __ffsll((unsigned long long)hb) - 1);
        const int64_t rw = (int64_t)b * R + j;
        float lam = kNegInf, st = s;
        if (trunc) {
          lam = a.tinfo[rw].x;
          st = 0.0f;
          for (int c = l; c < nc; c += kWave) st += a.tpart[rw * nc + c];
          st = wave_sum(st);
        }
        // Where a draw at this row would land: x_j (j < d) is removed from
        // its chunk's weight for the one-hot residual; row d is the bonus.
        const float wx = (j < d && hb && lxv >= lam) ? fast_exp2((lxv - m) * kk) : 0.0f;
        const int cxw = (j < d) ? cx : -1;
        const float uK = sh.u[a.K];
        ChunkPick pk;
        if constexpr (slices) {
          // From the quarter sums: a chunk weighs the sum of its quarters',
          // and x_j leaves its quarter in the chunk's own frame (its term as
          // the stream pass formed it): a quarter holding nothing else but
          // x_j then weighs exactly 0.
          const int xq = (cxw >= 0 && hb)
                             ? (xj - cx * kChunk<DT>) / kVec<DT> / kThreads / 2
                             : -1;
          auto quarters = [&](int c) {
            const f32x4 qs = sh.wc[j * nc + c];
            const float mc = sh.pc[j * nc + c].x;
            const double sc = chunk_scale(mc, m, kk);
            double s0 = qs.x, s1 = qs.y, s2 = qs.z, s3 = qs.w;
            if (c == cxw) {
              const double wxr = fast_exp2((lxv - mc) * kk);
              s0 = xq == 0 ? fmax(0.0, s0 - wxr) : s0;
              s1 = xq == 1 ? fmax(0.0, s1 - wxr) : s1;
              s2 = xq == 2 ? fmax(0.0, s2 - wxr) : s2;
              s3 = xq == 3 ? fmax(0.0, s3 - wxr) : s3;
            }
            return QuarterW{s0 * sc, s1 * sc, s2 * sc, s3 * sc};
          };
          pk = pick_chunk_slice(nc, uK, quarters);
        } else {
          pk = pick_chunk(nc, uK, [&](int c) {
            double W;
            if (trunc) {
              W = a.tpart[rw * nc + c];
            } else {
              const f32x4 p = part(j, c);
              W = chunk_weight(p.y, p.x, m, kk);
            }
            return c == cxw ? fmax(0.0, W - (double)wx) : W;
          });
        }
        if (l == 0) {
          sh.m[j] = m;
          sh.s[j] = st;
          sh.su[j] = s;
          sh.lam[j] = lam;
          sh.lx[j] = lxv;
          sh.bad[j] = !(s > 0.0f) || !isfinite(s) || !isfinite(m);
          sh.pick[j] = pk;
        }
      }
    }
  };
  if (cached)
    combine_rows([&](int j, int c) { return sh.pc[j * nc + c]; });
  else
    combine_rows([&](int j, int c) { return load_partial(Pb + (int64_t)j * nc + c); });
  __syncthreads();
  // Draw rows: row 0 (the first draft rejected, or no drafts) and row d
  // (every draft accepted) are the likely ones. Their chosen chunks are
  // requested before the accept scan; another row's after it. With q given,
  // a rejection's draw is the residual kernels' work: only row d is drawn
  // here.
  // A row's pick takes either its chunk's quarter (rs) or the whole chunk
  // (raw).
  u32x4 raw[kLoads], rawd[kLoads], rs[kSliceLoads], rsd[kSliceLoads];
  auto load_pick = [&](int r, u32x4 (&full)[kLoads], u32x4 (&part)[kSliceLoads]) {
    if constexpr (slices)
      draw_load_slice<DT>(a, b, r, sh.pick[r], part);
    else
      draw_load<DT, VP>(a, b, r, sh.pick[r], full);
  };
  if (!greedy) {
    if constexpr (Q) {
      load_pick(d, raw, rs);
    } else {
      load_pick(0, raw, rs);
      if (d > 0) load_pick(d, rawd, rsd);
    }
  }
  // The accept scan. Every wavefront takes it (the same LDS inputs through
  // the same instructions: the same result), so that each can request the
  // draw row's chunk with no barrier in between; wavefront 0 writes the
  // outputs.
  int st = 0, x = -1;
  if (l < d) {
    x = sh.x[l];
    if (x < 0 || x >= a.V) st |= SS_ST_TOKEN_RANGE;
  }
  if (l <= d && sh.bad[l]) st |= SS_ST_NONFINITE;
  st = wave_or(st);
  bool acc = true;
  float px = -1.0f;
  if (!st && l < d) {
    if (greedy) {
      acc = (x == sh.idx[l]);
    } else {
      px = (sh.lx[l] >= sh.lam[l]) ? fast_exp2((sh.lx[l] - sh.m[l]) * kk) / sh.s[l]
                                   : 0.0f;
      const float qx = Q ? sh.qx[l] : 1.0f;
      acc = (qx > 0.0f) ? (sh.u[l] <= px / qx) : (px > 0.0f);
    }
  }
  // Wavefront scan of the accept flags: the first rejection ends the run.
  const unsigned long long rej = __ballot(!acc);
  const int ral = rej ? __ffsll((unsigned long long)rej) - 1 : d;
  if (!Q && !st && !greedy && ral > 0 && ral < d) load_pick(ral, raw, rs);
  if (w == 0) {
    if (st) {
      if (l == 0) {
        atomicOr(&a.status[b], st);
        sh.st = st;
        sh.acc_len = 0;
      }
    } else {
      const int al = ral;
      if (l < R) {
        int tok = -1;
        if (l < al)
          tok = x;
        else if (l == al && greedy)
          tok = sh.idx[l];
        if (!(l == al && !greedy)) a.out[(int64_t)b * R + l] = tok;
        sh.tok[l] = tok;
      }
      if (a.p_draft && l < a.K)
        a.p_draft[(int64_t)b * a.K + l] =
            (!greedy && l < d && l <= al) ? px : -1.0f;
      // Log-probabilities: accepted drafts here, a drawn token after its
      // draw. Greedy rows are at temperature 1 (an accepted draft and the
      // final token are the row's argmax: log p = -log s).
      if (a.logprob && l < R) {
        float lp = NAN;
        if (greedy && l <= al)
          lp = -logf(sh.s[l]);
        else if (!greedy && l < al)
          lp = ((sh.lx[l] - sh.m[l]) * kk - log2f(sh.su[l])) * kLn2;
        if (greedy || l != al) a.logprob[(int64_t)b * R + l] = lp;
      }
      if (l == 0) {
        a.nem[b] = al + 1;
        sh.acc_len = al;
        sh.st = 0;
      }
    }
  }
  // The automaton's header and last record, handed to wavefront 0 across the
  // barrier below: the record, requested after the first barrier, has had
  // the combine and the accept scan to arrive.
  if constexpr (SAM) {
    if (w == kSamWave && l < 8) {
      sh.hdr[l] = hv;
      if (l < 4) sh.rec[l] = rv;
    }
  }
  __syncthreads();
  if constexpr (SAM) {
    if (w == 0) {
      hv = (l < 8) ? sh.hdr[l] : 0;
      rv = (l < 4) ? sh.rec[l] : 0;
    }
  }
  const int al = sh.acc_len;
  const bool residual = Q && sh.st == 0 && !greedy && al < d;
  if (tid == 0) {
    a.seqinfo[b] = residual ? i32x4{al + 1, __float_as_int(sh.m[al]),
                                    __float_as_int(sh.s[al]), __float_as_int(kk)}
                            : i32x4{0, 0, 0, 0};
    if (residual)
      a.seqinfo2[b] = f32x4{sh.lam[al], sh.su[al], trunc ? 1.0f : 0.0f, 0.0f};
  }
  // Automaton step (wavefront 0): the emitted tokens sh.tok[0..al] are
  // appended in order; when a token is drawn, the accepted drafts before it
  // are appended while the draw's chunk is in flight (with none, the record
  // of link(last) is fetched then, for the drawn token's first lookups).
  bool whole = true, cs_ready = false;
  int appended = 0;
  const bool drawn = sh.st == 0 && !greedy && !residual;
  if (drawn) {
    const OneToken excl{(al < d) ? sh.x[al] : -1};
    if constexpr (SAM) {
      if (w == 0) {
        cs = cursor_from_lanes(hv, rv);
        cs_ready = true;
        if (al > 0) {
          whole = sam_append(S, cs, sh.tok, al, R, a.max_len);
          appended = al;
        } else {
          sam_cursor_fetch_link(S, cs);
        }
      }
    }
    // Row d's chunk is taken when it is the draw row: a copy, which waits
    // for it, so it comes after the automaton step.
    const ChunkPick pk = sh.pick[al];
    if (!Q && al == d && d > 0) {
      if constexpr (slices) {
#pragma unroll
        for (int it = 0; it < kSliceLoads; ++it) rs[it] = rsd[it];
      } else {
#pragma unroll
        for (int it = 0; it < kLoads; ++it) raw[it] = rawd[it];
      }
    }
    int tok;
    if constexpr (slices)
      tok = draw_in_chunk<DT, VP, false, OneToken, NoDuring, NoQ, true>(
          a, sh.draw, b, al, pk, excl, sh.m[al], kk, 0.0f, sh.lam[al], rs);
    else
      tok = draw_in_chunk<DT, VP, false>(a, sh.draw, b, al, pk, excl, sh.m[al], kk, 0.0f,
                                         sh.lam[al], raw);
    // (No barrier after this: the one reader of sh.tok[al], the automaton
    // step, runs in wavefront 0, as does the thread that writes it.)
    if (tid == 0) {
      a.out[(int64_t)b * R + al] = tok;
      sh.tok[al] = tok;
      if (a.logprob)
        a.logprob[(int64_t)b * R + al] =
            drawn_logprob<DT>(a, b, al, tok, sh.draw.result_l, sh.m[al], sh.su[al], kk);
    }
  }
  if constexpr (SAM) {
    if (w == 0) {
      int32_t* nd = a.next_draft + (int64_t)b * a.K;
      if (!cs_ready) cs = cursor_from_lanes(hv, rv);
      if (sh.st == 0 && whole)
        whole = sam_append(S, cs, sh.tok + appended, al + 1 - appended, R, a.max_len);
      if (whole)
        sam_draft_cursor(S, cs, a.K, nd, a.next_draft_len + b, a.next_match_len + b);
      else
        sam_draft_seq(S, a.K, nd, a.next_draft_len + b, a.next_match_len + b);
    }
  }
}

template <int DT, bool VP>
__global__ __launch_bounds__(kThreads) void verify_residual_sums(Args a) {
  __shared__ f32x4 red[kWaves];
  const int tid = threadIdx.x, w = tid / kWave, l = tid % kWave;
  const int nc = a.nchunks;
  const int b = blockIdx.x / nc;
  const int c = blockIdx.x - b * nc;
  const i32x4 info = a.seqinfo[b];
  if (info.x == 0) return;
  const int r = info.x - 1;
  const float m = __int_as_float(info.y), S = __int_as_float(info.z);
  const float kk = __int_as_float(info.w);
  const float lam = a.seqinfo2[b].x;
  const float invS = 1.0f / S;
  const int R = a.K + 1;
  const int cstart = c * kChunk<DT>;
  const unsigned char* rowp =
      a.logits + ((int64_t)b * R + r) * a.V * Dt<DT>::kBytes;
  const float* qrow = a.q + ((int64_t)b * a.K + r) * a.V;
  // The chunk's q and logits are all requested before either is used (past
  // the row's end the logits are -inf and q is 0: those terms are 0). q
  // goes first: requested after the logits, its loads were scheduled behind
  // the exps of the logits, a second round trip.
  QChunk<DT> qc;
  load_q_chunk<DT, VP>(qrow, cstart, a.V, tid, qc);
  u32x4 raw[kLoads];
  if constexpr (VP)
    load_chunk_flat<DT>(rowp, cstart, a.V, tid, raw);
  else
    load_chunk<DT, VP>(rowp, cstart, a.V, tid, raw);
  // (no instruction moves across this point: every load is requested before
  // the first result is used)
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (VP) chunk_tail_neginf<DT>(cstart, a.V, tid, raw);
  q_tail_zero<DT, VP>(cstart, a.V, tid, qc);
  // Summed per quarter of the chunk (loads 2q, 2q + 1), so that the draw
  // can re-read one quarter; the chunk's sum is (s0 + s1) + (s2 + s3).
  float sq[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float s = 0.0f;
#pragma unroll
    for (int it = 2 * q; it < 2 * q + 2; ++it)
#pragma unroll
      for (int k = 0; k < kVec<DT>; ++k) {
        const float v = elem<DT>(raw[it], k);
        const float wv = (v >= lam) ? fast_exp2((v - m) * kk) : 0.0f;
        s += fmaxf(0.0f, wv * invS - qc.at(it, k));
      }
    sq[q] = s;
  }
  wave_inclusive_sum_n(sq);
  if (l == kWave - 1) red[w] = f32x4{sq[0], sq[1], sq[2], sq[3]};
  __syncthreads();
  if (tid == 0) {
    f32x4 t = red[0];
    for (int i = 1; i < kWaves; ++i) t = f32x4{t.x + red[i].x, t.y + red[i].y,
                                               t.z + red[i].z, t.w + red[i].w};
    a.rpart[(int64_t)b * nc + c] = (t.x + t.y) + (t.z + t.w);
    a.rqpart[(int64_t)b * nc + c] = t;
  }
}

template <int DT, bool VP>
__global__ __launch_bounds__(kThreads) void verify_residual_draw(Args a) {
  __shared__ ChunkPick pick_sh;
  __shared__ int from_p;
  __shared__ DrawShared dsh;
  const int tid = threadIdx.x, w = tid / kWave, l = tid % kWave;
  const int nc = a.nchunks;
  const int b = blockIdx.x;
  const i32x4 info = a.seqinfo[b];
  if (info.x == 0) return;
  const int r = info.x - 1;
  const float m = __int_as_float(info.y), S = __int_as_float(info.z);
  const float kk = __int_as_float(info.w);
  const f32x4 info2 = a.seqinfo2[b];
  const float lam = info2.x, Su = info2.y;
  const bool trunc = info2.z != 0.0f;
  const int R = a.K + 1;
  if (w == 0) {
    const float u = a.uniforms[(int64_t)b * R + a.K];
    const float* rp = a.rpart + (int64_t)b * nc;
    ChunkPick pk;
    if constexpr (VP) {
      // The quarter sums: the chunk, then its quarter (as the finalize picks).
      const f32x4* rq = a.rqpart + (int64_t)b * nc;
      auto quarters = [&](int c) {
        const f32x4 t = rq[c];
        return QuarterW{t.x, t.y, t.z, t.w};
      };
      pk = pick_chunk_slice(nc, u, quarters);
    } else {
      pk = pick_chunk(nc, u, [&](int c) { return load_f32(rp + c); });
    }
    // max(0, p - q) vanishes everywhere only when p == q: then draw from p.
    const bool fallback = pk.chunk < 0;
    if (fallback) {
      const int64_t rw = (int64_t)b * R + r;
      const f32x4* Pr = a.partials + rw * nc;
      pk = pick_chunk(nc, u, [&](int c) {
        if (trunc) return (double)load_f32(a.tpart + rw * nc + c);
        const f32x4 p = load_partial(Pr + c);
        return chunk_weight(p.y, p.x, m, kk);
      });
    }
    if (l == 0) {
      pick_sh = pk;
      from_p = fallback;
    }
  }
  __syncthreads();
  u32x4 raw[kLoads];
  int tok;
  if (from_p) {
    draw_load<DT, VP>(a, b, r, pick_sh, raw);
    tok = draw_in_chunk<DT, VP, false>(a, dsh, b, r, pick_sh, OneToken{-1}, m, kk, 0.0f,
                                       lam, raw);
  } else if constexpr (VP) {
    // One quarter of the chosen chunk: its q, then its logits, all requested
    // before either is used.
    QChunk<DT, kSliceLoads> qc;
    u32x4 rs[kSliceLoads];
    if (pick_sh.chunk >= 0) {
      const int cstart = pick_sh.chunk * kChunk<DT>;
      load_q_slice<DT>(a.q + ((int64_t)b * a.K + r) * a.V, cstart, a.V, pick_sh.slice, qc);
      draw_load_slice<DT>(a, b, r, pick_sh, rs);
      __builtin_amdgcn_sched_barrier(0);
      q_slice_tail_zero<DT>(cstart, a.V, pick_sh.slice, qc);
    }
    tok = draw_in_chunk<DT, VP, true, OneToken, NoDuring, QChunk<DT, kSliceLoads>, true>(
        a, dsh, b, r, pick_sh, OneToken{-1}, m, kk, 1.0f / S, lam, rs, NoDuring{}, qc);
  } else {
    // (q first, as in the residual sums)
    QChunk<DT> qc;
    if (pick_sh.chunk >= 0) {
      const int cstart = pick_sh.chunk * kChunk<DT>;
      load_q_chunk<DT, VP>(a.q + ((int64_t)b * a.K + r) * a.V, cstart, a.V, tid, qc);
      const unsigned char* rowp = a.logits + ((int64_t)b * R + r) * a.V * Dt<DT>::kBytes;
      if constexpr (VP)
        load_chunk_flat<DT, false>(rowp, cstart, a.V, tid, raw);
      else
        load_chunk<DT, VP, false>(rowp, cstart, a.V, tid, raw);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (VP) chunk_tail_neginf<DT>(cstart, a.V, tid, raw);
      q_tail_zero<DT, VP>(cstart, a.V, tid, qc);
    }
    tok = draw_in_chunk<DT, VP, true>(a, dsh, b, r, pick_sh, OneToken{-1}, m, kk,
                                      1.0f / S, lam, raw, NoDuring{}, qc);
  }
  if (tid == 0) {
    a.out[(int64_t)b * R + r] = tok;
    if (a.logprob)
      a.logprob[(int64_t)b * R + r] =
          drawn_logprob<DT>(a, b, r, tok, dsh.result_l, m, Su, kk);
  }
}

// ---------------------------------------------------------------------------
// Workspace layout (bytes, each region 256-byte aligned).
// ---------------------------------------------------------------------------
struct WsLayout {
  size_t partials, wparts, seqinfo, seqinfo2, rpart, rqpart;
  // truncation (top-k / top-p) regions; zero-sized without it
  size_t hist, hhdr, cand, tpart, tinfo;
  size_t total;
};

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

inline int nchunks_for(int V, int dtype) {
  const int ch = dtype == SS_DTYPE_F32 ? kChunk<SS_DTYPE_F32> : kChunk<SS_DTYPE_BF16>;
  return (V + ch - 1) / ch;
}

WsLayout ws_layout(int B, int K, int V, bool trunc) {
  const size_t nc = (size_t)nchunks_for(V, SS_DTYPE_F32);  // the larger count
  const size_t rows = (size_t)B * (K + 1);
  WsLayout L;
  size_t o = 0;
  auto take = [&](size_t& at, size_t bytes) {
    at = o;
    o = align256(o + bytes);
  };
  take(L.partials, rows * nc * sizeof(f32x4));
  take(L.wparts, rows * nc * sizeof(f32x4));
  take(L.seqinfo, (size_t)B * sizeof(i32x4));
  take(L.seqinfo2, (size_t)B * sizeof(f32x4));
  take(L.rpart, (size_t)B * nc * sizeof(float));
  take(L.rqpart, (size_t)B * nc * sizeof(f32x4));
  const size_t t = trunc ? 1 : 0;
  take(L.hist, t * rows * nc * kHistBins * sizeof(unsigned long long));
  take(L.hhdr, t * rows * nc * sizeof(i32x4));
  take(L.cand, t * rows * nc * std::min(kSegCap, V) * sizeof(float));
  take(L.tpart, t * rows * nc * sizeof(float));
  take(L.tinfo, t * rows * sizeof(f32x4));
  L.total = o;
  return L;
}

template <int DT, bool VP, bool SAM, bool SL>
void launch_finalize(const Args& a, hipStream_t s) {
  if (a.q)
    hipLaunchKernelGGL((spec_finalize_kernel<DT, VP, false, true, SL>), dim3((unsigned)a.B),
                       dim3(kThreads), 0, s, a);
  else
    hipLaunchKernelGGL((spec_finalize_kernel<DT, VP, SAM, false, SL>), dim3((unsigned)a.B),
                       dim3(kThreads), 0, s, a);
}

template <int DT, bool VP, bool SAM>
int launch_finish(const Args& a, hipStream_t s) {
  // Quarters: their sums exist (vector path), no row truncates, and every
  // row's partials fit the finalize's cache.
  const bool sl = VP && a.wparts != nullptr && a.tinfo == nullptr &&
                  (a.K + 1) * a.nchunks <= kPartialCache;
  if (sl)
    launch_finalize<DT, VP, SAM, true>(a, s);
  else
    launch_finalize<DT, VP, SAM, false>(a, s);
  int rc = check_launch("spec_finish");
  if (rc != SS_OK || a.q == nullptr) return rc;
  hipLaunchKernelGGL((verify_residual_sums<DT, VP>),
                     dim3((unsigned)((int64_t)a.B * a.nchunks)), dim3(kThreads), 0, s,
                     a);
  rc = check_launch("spec_finish residual sums");
  if (rc != SS_OK) return rc;
  hipLaunchKernelGGL((verify_residual_draw<DT, VP>), dim3((unsigned)a.B),
                     dim3(kThreads), 0, s, a);
  return check_launch("spec_finish residual draw");
}

// Which passes to launch.
enum Passes { kStream = 1, kFinish = 2 };

int run(int passes, const void* logits, int dtype, int B, int K, int V,
        const int32_t* draft, const int32_t* draft_len, const float* q,
        const float* temperature, const float* uniforms, const int32_t* top_k,
        const float* top_p, int32_t* out_tokens,
        int32_t* num_emitted, float* p_draft, float* logprob, int32_t* status,
        void* workspace, size_t ws_bytes, void* sam_state, int max_len,
        int32_t* next_draft,
        int32_t* next_draft_len, int32_t* next_match_len, void* stream,
        const char* fn) {
  if (B < 1 || K < 1 || K > SS_MAX_K || V < 1 || V > kMaxV)
    return set_error(SS_EINVAL,
                     "%s: need B >= 1, 1 <= K <= %d, 1 <= V <= %d "
                     "(got B=%d K=%d V=%d)",
                     fn, SS_MAX_K, kMaxV, B, K, V);
  if (dtype != SS_DTYPE_F32 && dtype != SS_DTYPE_BF16)
    return set_error(SS_EINVAL, "%s: unknown dtype %d", fn, dtype);
  if (!logits || !draft || !draft_len || !temperature || !workspace)
    return set_error(SS_EINVAL, "%s: a required pointer is NULL", fn);
  if ((passes & kFinish) && (!out_tokens || !num_emitted || !status))
    return set_error(SS_EINVAL, "%s: an output pointer is NULL", fn);
  if ((uintptr_t)workspace & 255)
    return set_error(SS_EINVAL, "%s: workspace must be 256-byte aligned", fn);
  if (((uintptr_t)logits & 15) || ((uintptr_t)q & 15))
    return set_error(SS_EINVAL, "%s: logits and q must start on a 16-byte boundary",
                     fn);
  if (sam_state) {
    if (((uintptr_t)sam_state & 255) || max_len < 1 || max_len > SS_MAX_LEN)
      return set_error(SS_EINVAL, "%s: state must be 256-byte aligned and "
                                  "1 <= max_len <= %d", fn, SS_MAX_LEN);
    if (q)
      return set_error(SS_EINVAL, "%s: the automaton step takes one-hot drafts "
                                  "(q must be NULL)", fn);
    if (!next_draft || !next_draft_len || !next_match_len)
      return set_error(SS_EINVAL, "%s: next-draft outputs must be non-null", fn);
    if (next_draft == draft || next_draft_len == draft_len)
      return set_error(SS_EINVAL, "%s: next-draft outputs must not alias the "
                                  "drafts being verified", fn);
  }
  const bool trunc = top_k != nullptr || top_p != nullptr;
  const WsLayout L = ws_layout(B, K, V, trunc);
  if (ws_bytes < L.total)
    return set_error(SS_EWORKSPACE,
                     "%s: workspace %zu < %zu bytes%s", fn, ws_bytes, L.total,
                     trunc ? " (top_k / top_p need ss_verify_workspace_bytes_ex "
                             "with SS_WS_TRUNCATION)"
                           : "");
  unsigned char* ws = reinterpret_cast<unsigned char*>(workspace);
  Args a;
  a.logits = reinterpret_cast<const unsigned char*>(logits);
  a.B = B;
  a.K = K;
  a.V = V;
  a.nchunks = nchunks_for(V, dtype);
  a.draft = draft;
  a.draft_len = draft_len;
  a.dl_offset = 0;
  a.dl_status = SS_ST_DRAFT_LEN;
  a.q = q;
  a.temperature = temperature;
  a.uniforms = uniforms;
  a.out = out_tokens;
  a.nem = num_emitted;
  a.p_draft = p_draft;
  a.logprob = logprob;
  a.top_k = top_k;
  a.top_p = top_p;
  a.status = status;
  a.partials = reinterpret_cast<f32x4*>(ws + L.partials);
  a.wparts = reinterpret_cast<f32x4*>(ws + L.wparts);
  a.seqinfo = reinterpret_cast<i32x4*>(ws + L.seqinfo);
  a.seqinfo2 = reinterpret_cast<f32x4*>(ws + L.seqinfo2);
  a.rpart = reinterpret_cast<float*>(ws + L.rpart);
  a.rqpart = reinterpret_cast<f32x4*>(ws + L.rqpart);
  a.hist = trunc ? reinterpret_cast<unsigned long long*>(ws + L.hist) : nullptr;
  a.hhdr = trunc ? reinterpret_cast<i32x4*>(ws + L.hhdr) : nullptr;
  a.cand = trunc ? reinterpret_cast<float*>(ws + L.cand) : nullptr;
  a.segcap = std::min(kSegCap, V);
  a.tpart = trunc ? reinterpret_cast<float*>(ws + L.tpart) : nullptr;
  a.tinfo = trunc ? reinterpret_cast<f32x4*>(ws + L.tinfo) : nullptr;
  a.sam = reinterpret_cast<unsigned char*>(sam_state);
  a.max_len = max_len;
  a.sl = sam_layout(max_len > 0 ? max_len : 1);
  a.next_draft = next_draft;
  a.next_draft_len = next_draft_len;
  a.next_match_len = next_match_len;
  // Rows are 16-byte aligned when V is a multiple of the vector width (the
  // base is checked above); otherwise the element-wise loads are used.
  const int vec = dtype == SS_DTYPE_F32 ? 4 : 8;
  const bool vp = V % vec == 0;
  hipStream_t s = as_stream(stream);
  const bool f32 = dtype == SS_DTYPE_F32;
  int rc = SS_OK;
  if (passes & kStream) {
    rc = launch_stream(a, f32, vp, s);
    if (rc != SS_OK) return rc;
  }
  if (passes & kFinish) {
    if (trunc) {
      rc = launch_truncation(a, f32, vp, s);
      if (rc != SS_OK) return rc;
    }
    if (sam_state)
      rc = f32 ? (vp ? launch_finish<SS_DTYPE_F32, true, true>(a, s)
                     : launch_finish<SS_DTYPE_F32, false, true>(a, s))
               : (vp ? launch_finish<SS_DTYPE_BF16, true, true>(a, s)
                     : launch_finish<SS_DTYPE_BF16, false, true>(a, s));
    else
      rc = f32 ? (vp ? launch_finish<SS_DTYPE_F32, true, false>(a, s)
                     : launch_finish<SS_DTYPE_F32, false, false>(a, s))
               : (vp ? launch_finish<SS_DTYPE_BF16, true, false>(a, s)
                     : launch_finish<SS_DTYPE_BF16, false, false>(a, s));
  }
  return rc;
}

}  // namespace
}  // namespace specsam

using namespace specsam;

extern "C" size_t ss_verify_workspace_bytes_ex(int B, int K, int V, int flags) {
  if (B < 1 || K < 1 || K > SS_MAX_K || V < 1 || V > kMaxV) return 0;
  if (flags & ~SS_WS_TRUNCATION) return 0;
  return ws_layout(B, K, V, (flags & SS_WS_TRUNCATION) != 0).total;
}

extern "C" size_t ss_verify_workspace_bytes(int B, int K, int V) {
  return ss_verify_workspace_bytes_ex(B, K, V, 0);
}

extern "C" size_t ss_tree_workspace_bytes(int B, int N, int V) {
  if (B < 1 || N < 1 || N > SS_MAX_TREE || V < 1 || V > kMaxV) return 0;
  return ws_layout(B, N - 1, V, false).total;
}

extern "C" int spec_verify_tree(const void* logits, int dtype, int B, int N, int V,
                                const int32_t* tokens, const int32_t* parent,
                                const int32_t* n_nodes, const float* temperature,
                                const float* uniforms, int32_t* out_tokens,
                                int32_t* out_nodes, int32_t* num_emitted,
                                int32_t* status, void* workspace, size_t ws_bytes,
                                void* stream) {
  const char* fn = "spec_verify_tree";
  if (B < 1 || N < 1 || N > SS_MAX_TREE || V < 1 || V > kMaxV)
    return set_error(SS_EINVAL, "%s: need B >= 1, 1 <= N <= %d, 1 <= V <= %d "
                                "(got B=%d N=%d V=%d)", fn, SS_MAX_TREE, kMaxV, B, N, V);
  if (dtype != SS_DTYPE_F32 && dtype != SS_DTYPE_BF16)
    return set_error(SS_EINVAL, "%s: unknown dtype %d", fn, dtype);
  if (!logits || !tokens || !parent || !n_nodes || !temperature || !out_tokens ||
      !out_nodes || !num_emitted || !status || !workspace)
    return set_error(SS_EINVAL, "%s: a required pointer is NULL", fn);
  if ((uintptr_t)workspace & 255)
    return set_error(SS_EINVAL, "%s: workspace must be 256-byte aligned", fn);
  if ((uintptr_t)logits & 15)
    return set_error(SS_EINVAL, "%s: logits must start on a 16-byte boundary", fn);
  const WsLayout L = ws_layout(B, N - 1, V, false);
  if (ws_bytes < L.total)
    return set_error(SS_EWORKSPACE, "%s: workspace %zu < %zu bytes", fn, ws_bytes,
                     L.total);
  unsigned char* ws = reinterpret_cast<unsigned char*>(workspace);
  Args a{};
  a.logits = reinterpret_cast<const unsigned char*>(logits);
  a.B = B;
  a.K = N - 1;  // rows per sequence: N, of which n_nodes[b] are read
  a.V = V;
  a.nchunks = nchunks_for(V, dtype);
  a.draft = nullptr;
  a.draft_len = n_nodes;
  a.dl_offset = -1;
  a.dl_status = SS_ST_TREE;
  a.temperature = temperature;
  a.uniforms = uniforms;
  a.out = out_tokens;
  a.nem = num_emitted;
  a.status = status;
  a.partials = reinterpret_cast<f32x4*>(ws + L.partials);
  a.wparts = reinterpret_cast<f32x4*>(ws + L.wparts);
  a.seqinfo = reinterpret_cast<i32x4*>(ws + L.seqinfo);
  a.seqinfo2 = reinterpret_cast<f32x4*>(ws + L.seqinfo2);
  a.rpart = reinterpret_cast<float*>(ws + L.rpart);
  const int vec = dtype == SS_DTYPE_F32 ? 4 : 8;
  const bool vp = V % vec == 0;
  const bool f32 = dtype == SS_DTYPE_F32;
  hipStream_t s = as_stream(stream);
  int rc = launch_stream(a, f32, vp, s);
  if (rc != SS_OK) return rc;
  return launch_tree_finalize(a, f32, vp, tokens, parent, out_nodes, s);
}

extern "C" int spec_verify(const void* logits, int dtype, int B, int K, int V,
                           const int32_t* draft, const int32_t* draft_len,
                           const float* q, const float* temperature,
                           const float* uniforms, const int32_t* top_k,
                           const float* top_p, int32_t* out_tokens,
                           int32_t* num_emitted, float* p_draft, float* logprobs,
                           int32_t* status, void* workspace, size_t ws_bytes,
                           void* stream) {
  return run(kStream | kFinish, logits, dtype, B, K, V, draft, draft_len, q,
             temperature, uniforms, top_k, top_p, out_tokens, num_emitted, p_draft,
             logprobs, status, workspace, ws_bytes, nullptr, 0, nullptr, nullptr,
             nullptr, stream, "spec_verify");
}

extern "C" int spec_step(const void* logits, int dtype, int B, int K, int V,
                         const int32_t* draft, const int32_t* draft_len,
                         const float* temperature, const float* uniforms,
                         const int32_t* top_k, const float* top_p,
                         void* sam_state, int max_len, int32_t* out_tokens,
                         int32_t* num_emitted, float* p_draft, float* logprobs,
                         int32_t* status, int32_t* next_draft,
                         int32_t* next_draft_len, int32_t* next_match_len,
                         void* workspace, size_t ws_bytes, void* stream) {
  if (!sam_state)
    return set_error(SS_EINVAL, "spec_step: state is NULL");
  return run(kStream | kFinish, logits, dtype, B, K, V, draft, draft_len,
             nullptr, temperature, uniforms, top_k, top_p, out_tokens, num_emitted,
             p_draft, logprobs, status, workspace, ws_bytes, sam_state, max_len,
             next_draft, next_draft_len, next_match_len, stream, "spec_step");
}

extern "C" int spec_stream(const void* logits, int dtype, int B, int K, int V,
                           const int32_t* draft, const int32_t* draft_len,
                           const float* temperature, const float* uniforms,
                           const int32_t* top_k, const float* top_p,
                           void* workspace, size_t ws_bytes, void* stream) {
  return run(kStream, logits, dtype, B, K, V, draft, draft_len, nullptr,
             temperature, uniforms, top_k, top_p, nullptr, nullptr, nullptr,
             nullptr, nullptr, workspace, ws_bytes, nullptr, 0, nullptr, nullptr,
             nullptr, stream, "spec_stream");
}

extern "C" int spec_finish(const void* logits, int dtype, int B, int K, int V,
                           const int32_t* draft, const int32_t* draft_len,
                           const float* q, const float* temperature,
                           const float* uniforms, const int32_t* top_k,
                           const float* top_p, int32_t* out_tokens,
                           int32_t* num_emitted, float* p_draft, float* logprobs,
                           int32_t* status, void* sam_state, int max_len,
                           int32_t* next_draft, int32_t* next_draft_len,
                           int32_t* next_match_len, void* workspace,
                           size_t ws_bytes, void* stream) {
  return run(kFinish, logits, dtype, B, K, V, draft, draft_len, q, temperature,
             uniforms, top_k, top_p, out_tokens, num_emitted, p_draft, logprobs,
             status, workspace, ws_bytes, sam_state, max_len, next_draft,
             next_draft_len, next_match_len, stream, "spec_finish");
}

// ---------------------------------------------------------------------------
// spec_step_noalloc: spec_step whose workspace is the library's own device
// array, for callers that cannot allocate. Each GPU holds its own copy of
// the array (for the life of the process); its address on a device is taken
// once, with that device current, and kept. The workspace needs no
// initialisation (every region is written before it is read in the same
// call), so nothing is cleared between calls; calls that overlap on one GPU
// share the array and race.
// ---------------------------------------------------------------------------
namespace specsam {
namespace {

__device__ __align__(256) unsigned char scratch[SS_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

// The address of `scratch` on the current device.
int scratch_on_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return set_error(SS_ELAUNCH, "spec_step_noalloc: hipGetDevice: %s",
                     hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return set_error(SS_EINVAL, "spec_step_noalloc: device %d beyond %d", dev,
                     kMaxDevices);
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr)
        return set_error(SS_ELAUNCH, "spec_step_noalloc: hipGetSymbolAddress: %s",
                         hipGetErrorString(e));
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return SS_OK;
}

}  // namespace
}  // namespace specsam

extern "C" int spec_step_noalloc(const void* logits, int dtype, int B, int K, int V,
                                 const int32_t* draft, const int32_t* draft_len,
                                 const float* temperature, const float* uniforms,
                                 const int32_t* top_k, const float* top_p,
                                 void* sam_state, int max_len, int32_t* out_tokens,
                                 int32_t* num_emitted, float* p_draft, float* logprobs,
                                 int32_t* status, int32_t* next_draft,
                                 int32_t* next_draft_len, int32_t* next_match_len,
                                 void* stream) {
  const char* fn = "spec_step_noalloc";
  if (!sam_state) return set_error(SS_EINVAL, "%s: state is NULL", fn);
  if (B < 1 || K < 1 || K > SS_MAX_K || V < 1 || V > kMaxV)
    return set_error(SS_EINVAL,
                     "%s: need B >= 1, 1 <= K <= %d, 1 <= V <= %d "
                     "(got B=%d K=%d V=%d)",
                     fn, SS_MAX_K, kMaxV, B, K, V);
  const bool trunc = top_k != nullptr || top_p != nullptr;
  const size_t need = ws_layout(B, K, V, trunc).total;
  if (need > (size_t)SS_SCRATCH_BYTES)
    return set_error(SS_EWORKSPACE,
                     "%s: B=%d K=%d V=%d%s needs %zu bytes of scratch, more than "
                     "the %zu it holds",
                     fn, B, K, V, trunc ? " with top_k / top_p" : "", need,
                     (size_t)SS_SCRATCH_BYTES);
  void* ws = nullptr;
  const int rc = scratch_on_current_device(&ws);
  if (rc != SS_OK) return rc;
  return run(kStream | kFinish, logits, dtype, B, K, V, draft, draft_len, nullptr,
             temperature, uniforms, top_k, top_p, out_tokens, num_emitted, p_draft,
             logprobs, status, ws, (size_t)SS_SCRATCH_BYTES, sam_state, max_len,
             next_draft, next_draft_len, next_match_len, stream, fn);
}
