// Device-side suffix automaton: layout, Blumer extension and drafting, shared
// by the stand-alone automaton kernels (sam.hip) and the fused step kernel
// (verify.hip).
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
//           hash_slots, magic, ...
//   states  int4[2*max_len]: (len, link, min_endpos, first_edge); one 16-byte
//           load brings every field a step of the construction reads.
//   text    int32[max_len]: committed tokens (the draft source).
//   hash    int4[hash_slots]: (src, token, dst, next) open-addressing table
//           keyed by (src, token), in 128-byte buckets of 8 rows probed
//           linearly; `next` chains a state's transitions so a clone can copy
//           them. hash_slots = next power of two >= 6*max_len keeps the load
//           at most 1/2 for the at most 3*max_len transitions.
//
// Execution: one wavefront per sequence. The construction is a chain of
// dependent loads, so lanes do not split it; they cooperate on each hash
// probe (8 lanes read a whole bucket in one request, a ballot finds the key or
// the first empty row), and the next state record is loaded alongside each
// probe. Every lane performs the same stores with the same values, so each
// lane reads its own writes (no cross-lane ordering through memory is
// assumed).
#pragma once

#include "internal.h"

namespace specsam {

constexpr int kBucket = 8;  // rows per 128-byte bucket
constexpr int kSamMagic = 0x53414d31;

struct SamLayout {
  size_t states, text, slots, block;
  int hash_slots;
};

__host__ __device__ inline size_t sam_al256(size_t x) {
  return (x + 255) & ~(size_t)255;
}

__host__ __device__ inline SamLayout sam_layout(int max_len) {
  SamLayout L;
  const size_t want = (size_t)6 * (size_t)max_len;
  size_t h = 64;
  while (h < want) h <<= 1;
  L.hash_slots = (int)h;
  L.states = 64;
  L.text = L.states + (size_t)2 * max_len * 16;
  L.slots = sam_al256(L.text + (size_t)max_len * 4);
  L.block = sam_al256(L.slots + h * 16);
  return L;
}

enum SamHdr { H_N = 0, H_LAST, H_STATES, H_EDGES, H_STATUS, H_MAXLEN, H_V,
              H_SLOTS, H_MAGIC };

struct SamSeq {
  int* hdr;
  i32x4* st;
  int* text;
  i32x4* slots;
};

__device__ __forceinline__ SamSeq sam_seq(unsigned char* base, int b,
                                          const SamLayout& L) {
  unsigned char* p = base + (size_t)b * L.block;
  return SamSeq{reinterpret_cast<int*>(p), reinterpret_cast<i32x4*>(p + L.states),
                reinterpret_cast<int*>(p + L.text),
                reinterpret_cast<i32x4*>(p + L.slots)};
}

__device__ __forceinline__ unsigned sam_bucket(int s, int c, unsigned bmask) {
  unsigned long long k = ((unsigned long long)(unsigned)s << 32) | (unsigned)c;
  k ^= k >> 33;
  k *= 0xff51afd7ed558ccdull;
  k ^= k >> 33;
  k *= 0xc4ceb9fe1a85ec53ull;
  k ^= k >> 33;
  return (unsigned)k & bmask;
}

struct SamProbe {
  int slot;  // row of (s, c), or the first empty row in probe order; -1 if full
  bool found;
  int dst;
  int buckets;  // 128-byte buckets read
};

// Work counters of the extension (measurement builds of the kernels only;
// the counting template parameter is false on the normal path).
enum SamStat {
  SS_STAT_TOKENS = 0,    // tokens appended
  SS_STAT_PROBES,        // hash lookups (each one or more bucket reads)
  SS_STAT_BUCKETS,       // 128-byte buckets read by those lookups
  SS_STAT_WALK,          // suffix-link steps that inserted a transition
  SS_STAT_CLONES,        // states cloned
  SS_STAT_COPIED,        // transitions copied into clones
  SS_STAT_REDIRECTS,     // transitions redirected to clones
  SS_STAT_COUNT
};

struct SamCounters {
  unsigned long long v[SS_STAT_COUNT];
};

// Wave-cooperative lookup of (s, c). Uniform in, uniform out.
__device__ __forceinline__ SamProbe sam_probe(const i32x4* slots, unsigned bmask,
                                              int s, int c) {
  const int l = lane_id();
  unsigned bk = sam_bucket(s, c, bmask);
  for (unsigned it = 0; it <= bmask; ++it) {
    i32x4 v = i32x4{-2, -2, -2, -2};
    if (l < kBucket) v = slots[(size_t)bk * kBucket + l];
    const bool m = (l < kBucket) && v.x == s && v.y == c;
    const bool e = (l < kBucket) && v.x == -1;
    const unsigned long long bal = __ballot(m || e);
    if (bal) {
      const int f = __ffsll((unsigned long long)bal) - 1;
      SamProbe r;
      r.slot = (int)(bk * kBucket) + f;
      r.found = (__ballot(m) >> f) & 1ull;
      r.dst = __builtin_amdgcn_readlane(v.z, f);
      r.buckets = (int)it + 1;
      return r;
    }
    bk = (bk + 1) & bmask;
  }
  return SamProbe{-1, false, -1, (int)bmask + 1};
}

// Two lookups in one round trip, (s0, c) and (s1, c): lanes 0..7 read the
// first key's bucket, lanes 8..15 the second's. A lookup whose bucket holds
// neither its key nor an empty row is left unresolved (slot -2) for
// sam_probe to finish.
struct SamProbe2 {
  SamProbe a, b;
};

__device__ __forceinline__ SamProbe2 sam_probe2(const i32x4* slots, unsigned bmask,
                                                int s0, int s1, int c) {
  const int l = lane_id();
  const unsigned bk0 = sam_bucket(s0, c, bmask), bk1 = sam_bucket(s1, c, bmask);
  const bool second = l >= kBucket;
  const int s = second ? s1 : s0;
  const unsigned bk = second ? bk1 : bk0;
  i32x4 v = i32x4{-2, -2, -2, -2};
  if (l < 2 * kBucket) v = slots[(size_t)bk * kBucket + (l & (kBucket - 1))];
  const bool m = (l < 2 * kBucket) && v.x == s && v.y == c;
  const bool e = (l < 2 * kBucket) && v.x == -1;
  const unsigned long long bal = __ballot(m || e);
  const unsigned long long mb = __ballot(m);
  SamProbe2 r;
  SamProbe* out[2] = {&r.a, &r.b};
  const unsigned bks[2] = {bk0, bk1};
#pragma unroll
  for (int g = 0; g < 2; ++g) {
    const unsigned long long gb = (bal >> (g * kBucket)) & ((1ull << kBucket) - 1);
    SamProbe x{-2, false, -1, 1};
    if (gb) {
      const int f = __ffsll((unsigned long long)gb) - 1;
      const int lane = g * kBucket + f;
      x.slot = (int)(bks[g] * kBucket) + f;
      x.found = (mb >> lane) & 1ull;
      x.dst = __builtin_amdgcn_readlane(v.z, lane);
    }
    *out[g] = x;
  }
  return r;
}

struct SamHdrRegs {
  int n, last, nstates, nedges, status, max_len, V, slots;
};

__device__ __forceinline__ SamHdrRegs sam_load_header(const SamSeq& S) {
  const i32x4 h0 = reinterpret_cast<const i32x4*>(S.hdr)[0];
  const i32x4 h1 = reinterpret_cast<const i32x4*>(S.hdr)[1];
  return SamHdrRegs{h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
}

__device__ __forceinline__ void sam_store_header(const SamSeq& S,
                                                 const SamHdrRegs& h) {
  reinterpret_cast<i32x4*>(S.hdr)[0] = i32x4{h.n, h.last, h.nstates, h.nedges};
  S.hdr[H_STATUS] = h.status;
}

// What a wavefront keeps in registers while it works on one sequence: the
// header, the record of the last state and, after an extension, the link of
// the last state with its record. Every record here is exact: each one is
// either loaded after the stores that could change it or is what was just
// stored.
struct SamCursor {
  SamHdrRegs h;
  i32x4 rlast;      // record of h.last
  int link;         // link(h.last), or -1 if not carried
  i32x4 rlink;      // its record
};

// Loads the header, then the record of the last state.
__device__ __forceinline__ SamCursor sam_open(const SamSeq& S) {
  SamCursor cs;
  cs.h = sam_load_header(S);
  cs.rlast = S.st[cs.h.last];
  cs.link = -1;
  return cs;
}

// A cursor assembled from values fetched one dword per lane: lane k of hv
// holds header word k (k < 8), lane k of rv word k of the last state's record
// (k < 4). Wave-uniform result.
__device__ __forceinline__ SamCursor cursor_from_lanes(int hv, int rv) {
  SamCursor cs;
  cs.h = SamHdrRegs{__builtin_amdgcn_readlane(hv, 0), __builtin_amdgcn_readlane(hv, 1),
                    __builtin_amdgcn_readlane(hv, 2), __builtin_amdgcn_readlane(hv, 3),
                    __builtin_amdgcn_readlane(hv, 4), __builtin_amdgcn_readlane(hv, 5),
                    __builtin_amdgcn_readlane(hv, 6), __builtin_amdgcn_readlane(hv, 7)};
  cs.rlast = i32x4{__builtin_amdgcn_readlane(rv, 0), __builtin_amdgcn_readlane(rv, 1),
                   __builtin_amdgcn_readlane(rv, 2), __builtin_amdgcn_readlane(rv, 3)};
  cs.link = -1;
  return cs;
}

// Loads the record of link(last) into a cursor that does not carry it, so
// that the next extension looks up (last, c) and (link(last), c) in one round
// trip (the fused step issues this while its draw is in flight).
__device__ __forceinline__ void sam_cursor_fetch_link(const SamSeq& S, SamCursor& cs) {
  if (cs.link < 0 && cs.rlast.y >= 0) {
    cs.rlink = S.st[cs.rlast.y];
    cs.link = cs.rlast.y;
  }
}

// Appends token c at position n (Blumer's online extension; `cur` is numbered
// before `clone`) and moves the cursor to cur. Returns false if a bound check
// trips.
template <bool COUNT = false>
__device__ inline bool sam_extend_one(const SamSeq& S, SamCursor& cs, int c,
                                      unsigned bmask, SamCounters* ctr = nullptr) {
  auto tally = [&](int k, int n) {
    if constexpr (COUNT) ctr->v[k] += (unsigned long long)n;
  };
  SamHdrRegs& h = cs.h;
  tally(SS_STAT_TOKENS, 1);
  const int i = h.n;
  const int cur = h.nstates++;
  const int lencur = cs.rlast.x + 1;
  S.st[cur] = i32x4{lencur, -1, i, -1};
  int p = h.last;
  i32x4 rp = cs.rlast;
  SamProbe pr;
  int guard = 0;
  bool walked = false;
  // When the cursor carries the record of link(last), (last, c) and
  // (link(last), c) are looked up in one round trip, with the record of the
  // next state on the walk. The second lookup ran before (last, c) was
  // inserted: it is repeated if that insertion took the empty row it found.
  if (cs.link >= 0 && cs.link == rp.y) {
    const int p1 = cs.link;
    const i32x4 rp1 = cs.rlink;
    const int p2 = rp1.y;
    i32x4 rp2 = i32x4{0, -1, -1, -1};
    if (p2 != -1) rp2 = S.st[p2];  // in flight with the two lookups
    const SamProbe2 two = sam_probe2(S.slots, bmask, p, p1, c);
    tally(SS_STAT_PROBES, 2);
    tally(SS_STAT_BUCKETS, 2);
    SamProbe r0 = two.a, r1 = two.b;
    if (r0.slot == -2) {
      r0 = sam_probe(S.slots, bmask, p, c);
      tally(SS_STAT_PROBES, 1);
      tally(SS_STAT_BUCKETS, r0.buckets);
    }
    if (r0.slot < 0) return false;
    if (r0.found) {
      pr = r0;
      walked = true;
    } else {
      tally(SS_STAT_WALK, 1);
      S.slots[r0.slot] = i32x4{p, c, cur, rp.w};
      reinterpret_cast<int*>(&S.st[p])[3] = r0.slot;
      h.nedges++;
      if (r1.slot == -2 || (!r1.found && r1.slot == r0.slot)) {
        r1 = sam_probe(S.slots, bmask, p1, c);
        tally(SS_STAT_PROBES, 1);
        tally(SS_STAT_BUCKETS, r1.buckets);
      }
      if (r1.slot < 0) return false;
      p = p1;
      rp = rp1;
      if (r1.found) {
        pr = r1;
        walked = true;
      } else {
        tally(SS_STAT_WALK, 1);
        S.slots[r1.slot] = i32x4{p, c, cur, rp.w};
        reinterpret_cast<int*>(&S.st[p])[3] = r1.slot;
        h.nedges++;
        p = p2;
        rp = rp2;
        walked = (p == -1);
      }
    }
  }
  // Walk suffix links from p, adding (p, c) -> cur until (p, c) exists.
  while (!walked) {
    const int nxt = rp.y;
    i32x4 rn = i32x4{0, -1, -1, -1};
    if (nxt != -1) rn = S.st[nxt];  // in flight together with the probe
    pr = sam_probe(S.slots, bmask, p, c);
    tally(SS_STAT_PROBES, 1);
    tally(SS_STAT_BUCKETS, pr.buckets);
    if (pr.slot < 0) return false;
    if (pr.found) break;
    tally(SS_STAT_WALK, 1);
    S.slots[pr.slot] = i32x4{p, c, cur, rp.w};
    reinterpret_cast<int*>(&S.st[p])[3] = pr.slot;
    h.nedges++;
    p = nxt;
    if (p == -1) break;
    rp = rn;
    if (++guard > h.nstates) return false;
  }
  int link;
  i32x4 rlink;
  if (p == -1) {
    link = 0;
    rlink = i32x4{0, -1, 0, 0};  // not the root's record: not carried below
  } else {
    const int q = pr.dst;
    const i32x4 rq = S.st[q];
    if (rp.x + 1 == rq.x) {
      link = q;
      rlink = rq;  // loaded after the walk's stores; nothing below changes it
    } else {
      const int clone = h.nstates++;
      tally(SS_STAT_CLONES, 1);
      // Copy q's transitions into the clone. The next row of q's chain is
      // requested together with each probe (a probe ends at an empty row,
      // never at a row of the chain, so the read is not overtaken by the
      // store that follows).
      int first = -1, e = rq.w, g2 = 0;
      i32x4 se = i32x4{-1, -1, -1, -1};
      if (e != -1) se = S.slots[e];
      while (e != -1) {
        const int en = se.w;
        i32x4 sn = i32x4{-1, -1, -1, -1};
        if (en != -1) sn = S.slots[en];
        const SamProbe pc = sam_probe(S.slots, bmask, clone, se.y);
        tally(SS_STAT_PROBES, 1);
        tally(SS_STAT_BUCKETS, pc.buckets);
        tally(SS_STAT_COPIED, 1);
        if (pc.slot < 0 || pc.found) return false;
        S.slots[pc.slot] = i32x4{clone, se.y, se.z, first};
        first = pc.slot;
        h.nedges++;
        e = en;
        se = sn;
        if (++g2 > h.nedges) return false;
      }
      const i32x4 rc = i32x4{rp.x + 1, rq.y, rq.z, first};
      S.st[clone] = rc;
      // Redirect (p', c) -> q to the clone along the suffix path from p.
      int sl = pr.slot;
      i32x4 rr = rp;
      int g3 = 0;
      while (true) {
        reinterpret_cast<int*>(&S.slots[sl])[2] = clone;
        tally(SS_STAT_REDIRECTS, 1);
        const int pp = rr.y;
        if (pp == -1) break;
        rr = S.st[pp];
        const SamProbe p3 = sam_probe(S.slots, bmask, pp, c);
        tally(SS_STAT_PROBES, 1);
        tally(SS_STAT_BUCKETS, p3.buckets);
        if (p3.slot < 0 || !p3.found || p3.dst != q) break;
        sl = p3.slot;
        if (++g3 > h.nstates) return false;
      }
      reinterpret_cast<int*>(&S.st[q])[1] = clone;
      link = clone;
      rlink = rc;
    }
  }
  reinterpret_cast<int*>(&S.st[cur])[1] = link;
  h.last = cur;
  S.text[i] = c;
  h.n = i + 1;
  cs.rlast = i32x4{lencur, link, i, -1};
  // The cursor carries link(cur)'s record only when it is exact: after a walk
  // to the root (link 0) the root's record (its first transition) was not
  // loaded, and the next extension must not insert with it.
  cs.link = (p == -1) ? -1 : link;
  cs.rlink = rlink;
  return true;
}

// Appends tokens tk[0..cnt) (wave-uniform) to one sequence, stopping at the
// first token that is out of range or would exceed capacity. A sequence whose
// status is already non-zero is left alone. Returns false if the cursor no
// longer describes the sequence (an extension stopped part-way). Executed by
// one whole wavefront.
template <bool COUNT = false>
__device__ inline bool sam_append(const SamSeq& S, SamCursor& cs, const int32_t* tk,
                                  int cnt, int ld, int max_len,
                                  SamCounters* ctr = nullptr) {
  SamHdrRegs& h = cs.h;
  if (h.status != 0) return true;
  const unsigned bmask = (unsigned)(h.slots / kBucket) - 1u;
  int st = 0;
  bool whole = true;
  if (cnt < 0 || cnt > ld) {
    st = SS_ST_COUNT;
  } else {
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
      if (!sam_extend_one<COUNT>(S, cs, c, bmask, ctr)) {
        st = SS_ST_SAM_CAPACITY;
        whole = false;
        break;
      }
    }
  }
  h.status |= st;
  sam_store_header(S, h);
  return whole;
}

// Draft from state s with record rs: follow suffix links while the state has
// no outgoing transition, then lanes j < K gather text[p + 1 + j] where p is
// the min_endpos of the state reached. Executed by one whole wavefront.
__device__ inline void sam_draft_from(const SamSeq& S, int n, int nstates, int s,
                                      i32x4 rs, int K, int32_t* draft,
                                      int32_t* draft_len, int32_t* match_len) {
  // The walk ends at the root without loading its record: its length is 0,
  // which gives no draft.
  for (int g = 0; s > 0 && rs.w == -1 && g < nstates; ++g) {
    s = rs.y;
    if (s > 0) rs = S.st[s];
  }
  const int Lm = (s <= 0) ? 0 : rs.x;
  const int p = rs.z;
  const int d = (Lm == 0) ? 0 : min(K, n - 1 - p);
  const int l = lane_id();
  if (l < K) draft[l] = (l < d) ? S.text[p + 1 + l] : -1;
  if (l == 0) {
    *draft_len = d;
    *match_len = Lm;
  }
}

// Draft for one sequence from its stored header (the link walk starts at the
// last state).
__device__ inline void sam_draft_seq(const SamSeq& S, int K, int32_t* draft,
                                     int32_t* draft_len, int32_t* match_len) {
  const SamCursor cs = sam_open(S);
  sam_draft_from(S, cs.h.n, cs.h.nstates, cs.h.last, cs.rlast, K, draft, draft_len,
                 match_len);
}

// Draft from a cursor: after an extension the last state is the newest one,
// which has no outgoing transition, so the walk starts at its link, whose
// record the extension carried.
__device__ inline void sam_draft_cursor(const SamSeq& S, const SamCursor& cs, int K,
                                        int32_t* draft, int32_t* draft_len,
                                        int32_t* match_len) {
  if (cs.link >= 0 && cs.rlast.w == -1)
    sam_draft_from(S, cs.h.n, cs.h.nstates, cs.link, cs.rlink, K, draft, draft_len,
                   match_len);
  else
    sam_draft_from(S, cs.h.n, cs.h.nstates, cs.h.last, cs.rlast, K, draft,
                   draft_len, match_len);
}

}  // namespace specsam
