// Stream pass of the batched verification: reads every logit row a sequence
// needs once, in 32 KiB chunks, and leaves one partial per (row, chunk).
//
// Method ([P2] m.nxbn.cn guide §2.2; [P3] gogongxt notes "贪婪采样",
// "拒绝采样"): row j of sequence b is needed iff j <= draft_len[b] (rows past
// the drafts are never read). At T = 0 a partial is (max, lowest index of the
// max, NaN flag); at T > 0 it is (max m, sum of exp2((l - m) * log2e / T))
// plus the logit of the draft token x_j when x_j falls in the chunk, and the
// sum is also left per quarter of the chunk (the draws re-read one quarter).
// The finish pass combines them. When the request truncates its
// target (top-k / top-p), each chunk of a row at T > 0 also leaves a window
// histogram of its logits and copies the logits of a band of its bins (the
// ones that probably hold the row's threshold) to its candidate segment, for
// the selection kernel (trunc.hip).
//
// Design for gfx950: 256-thread workgroups each hold one chunk in registers
// (8 non-temporal 16-byte loads in flight per lane, each wavefront load one
// contiguous 1 KiB request) and write one 16-byte partial per row: nothing
// but loads, arithmetic and one store. The grid is (sequence, row lane,
// chunk): lane q of a sequence streams its chunk of rows q, q + G, q + 2G,
// ... up to the sequence's draft length. Launches whose row 0 alone gives
// fewer than 4096 workgroups (and draft trees, and launches that truncate)
// take G = K + 1, a workgroup per needed (row, chunk); larger ones take
// G = 2 for K <= 3 and 4 above,
// so that a sequence with no drafts leaves few idle workgroups per chunk
// (they read its draft length and leave) while drafted rows still spread
// over several workgroups.
#include <algorithm>

#include "stream_row.h"

namespace specsam {
namespace {

// Occupancy hint, for the histogram variant on the 16-byte load path only:
// 5 (fp32) or 3 (bf16) waves per SIMD. Under a hint of 6 the fp32 code
// spills a few registers to scratch, and the reloads, each a memory round
// trip, cost more than the extra wavefront gains (B = 256, V = 151936, no
// drafts, top-p: 56.4 us at 5 against 63.0 at 6). The plain variant takes
// none: the compiler then schedules it with 110 registers (4 waves per
// SIMD; 90 before the next row's loads were moved into the row, which that
// move more than repays), and such code streamed faster once many rows are
// needed than the 61 registers (8 waves) a hint of 6 gives (B = 256,
// V = 151936, K = 3, every draft full: 94.0 us against 97.5, equal with no
// drafts). The element-wise path takes none either: it would spill under
// one.
template <int DT, bool TR>
constexpr int kStreamWaves = (DT == SS_DTYPE_F32) ? 5 : 3;

// Row lanes G (see the file comment). Measured per launch at B = 256,
// V = 151936, fp32, K = 3 (events around 8 back-to-back launches, one MI355X):
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
  __shared__ f32x4 red[2 * kWaves + 1];
  __shared__ TrLds<TR> tl;
  TrShared* ts = nullptr;
  if constexpr (TR) ts = &tl.s;
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
  if (st) return;
  if constexpr (VP && !TR && DT == SS_DTYPE_F32) {
    // The lane's next row is requested as soon as this one's registers are
    // consumed, before its reductions and barriers: every row needed at
    // B = 256, K = 3 (two rows per lane) 96.4 -> 94.1 us per launch, c3
    // 28.4 -> 28.1 us. Only on the plain fp32 vector path: the other
    // variants would hold more registers across it, or spill (bf16's c4
    // launch, 32 x 5 rows: 6.78 -> 6.89 us).
    for (int j = q; j <= d; j += G) {
      if (j != 0 && j == q)
        load_chunk<DT, VP>(a.logits + ((int64_t)b * R + j) * a.V * Dt<DT>::kBytes,
                           cstart, a.V, tid, raw);
      if (j != q) x = draft_token(a, b, j);
      auto next = [&]() {
        if (j + G <= d)
          load_chunk<DT, VP>(a.logits + ((int64_t)b * R + j + G) * a.V * Dt<DT>::kBytes,
                             cstart, a.V, tid, raw);
      };
      stream_row<DT, VP, TR, true>(a, b, j, d, T, c, x, raw, red, ts, next);
    }
  } else {
    for (int j = q; j <= d; j += G) {
      if (j != 0)
        load_chunk<DT, VP>(a.logits + ((int64_t)b * R + j) * a.V * Dt<DT>::kBytes,
                           cstart, a.V, tid, raw);
      if (j != q) x = draft_token(a, b, j);
      stream_row<DT, VP, TR, true>(a, b, j, d, T, c, x, raw, red, ts, NoMid{});
    }
  }
}

// Draft trees: a tree's nodes usually all need their rows, so every
// (sequence, node, chunk) gets a workgroup (G = K + 1). So does a launch that
// may truncate rows: a truncated row's chunk takes several times the
// instructions of a plain one, and rows taken one after another in a
// workgroup leave the chip with too few loads in flight (B = 256,
// V = 151936, K = 3, top-k 50 then top-p 0.9, 882 of 1,024 rows needed:
// 142.4 us per launch against 160.7 with two lanes; top-p alone, 282 rows:
// 62.3 against 62.9).
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
  a.ngroups = (tree_rows(a) || a.hist) ? a.K + 1 : row_lanes(a.B, a.K, a.nchunks);
  return f32 ? (vp ? launch_stream_tr<SS_DTYPE_F32, true>(a, s)
                   : launch_stream_tr<SS_DTYPE_F32, false>(a, s))
             : (vp ? launch_stream_tr<SS_DTYPE_BF16, true>(a, s)
                   : launch_stream_tr<SS_DTYPE_BF16, false>(a, s));
}

}  // namespace specsam
