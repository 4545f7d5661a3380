// Top-k block selection: one workgroup selects for every row of a request.
//
// aisoku.org MiniMax-M3.1-Flash article, section "MSAの仕組み", and the
// agentlenshq page, section "MSA 実行プロセス" step 2 (local_blocks = 1): each
// row keeps its local block (the one holding the query token) plus the best
// of the other causal blocks, topk blocks in all.  Ties go to the lower block
// id; the kept ids are emitted ascending.  news.ainew.jp MI355X article,
// section 2: one workgroup per request covers all draft positions.
//
// Design: a row's candidates are spread over 1, 2 or 4 waves (4 / T when
// T < 4) and compared as 64-bit keys (orderable score << 32 | ~id, so a
// larger key is a better block and equal scores favour the lower id).  Each
// lane folds its candidates into its best key; the K1-th largest score
// word of a wave's lane maxima (K1 = topk - 1), as a key with zero low bits,
// has K1 real candidates at or above it, so only candidates reaching the
// largest such bound of the row's waves can be among the K1 best.  Those
// survivors (typically a few dozen) are gathered in LDS and ranked by
// counting; the winners are ordered by id.  A row with more
// survivors than LDS holds (a few lanes owning most of the best keys) falls
// back to per-lane sorted lists, wave-max pops and a merge-rank.  The kernel
// runs each path about once per launch, so code size (instruction fetch)
// counts as much as instruction count: loops stop at the wave's real
// candidate count instead of being duplicated per case.
#pragma once

#include "msa_device.h"

namespace msa {

constexpr int kMaxTopk = 16;
constexpr int kList = kMaxTopk - 1;  // per-lane list length (non-local picks)
constexpr int kBatch = 16;           // score loads in flight per lane

// One DPP step of a wave reduction: max with the lane the pattern names.
// Lanes outside `row_mask` see 0, the identity of an unsigned max, which
// lets the compiler fold the move into v_max_u32's DPP form.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_max_u32(uint32_t v) {
  const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, CTRL, ROW_MASK, 0xF, false);
  return o > v ? o : v;
}

// Wave-wide unsigned max, returned to every lane: DPP within rows of 16
// (quad swaps, half-row and row mirrors), row broadcasts across rows, then
// lane 63 holds the result.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_max_u32<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
  v = dpp_max_u32<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
  v = dpp_max_u32<0x141, 0xF>(v);  // row_half_mirror
  v = dpp_max_u32<0x140, 0xF>(v);  // row_mirror
  v = dpp_max_u32<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
  v = dpp_max_u32<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Wave-wide max of 64-bit keys: a 32-bit pass over the high words; when a
// single lane holds the high maximum its low word is read directly,
// otherwise a second pass runs over the low words of the tied lanes.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  const uint32_t vhi = (uint32_t)(v >> 32);
  const uint32_t hi = wave_max_u32(vhi);
  const uint64_t tied = __ballot(vhi == hi);
  uint32_t lo;
  if (__popcll(tied) == 1)
    lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, __builtin_ctzll(tied));
  else
    lo = wave_max_u32(vhi == hi ? (uint32_t)v : 0u);
  return ((uint64_t)hi << 32) | lo;
}

// Monotone map fp32 -> uint32 for a total order; NaN ranks as -inf and -0
// as +0.
__device__ __forceinline__ uint32_t orderable(float s) {
  if (s != s) s = -INFINITY;
  if (s == 0.f) s = 0.f;
  const uint32_t u = __builtin_bit_cast(uint32_t, s);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint64_t make_key(float s, int c) {
  return ((uint64_t)orderable(s) << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)c);
}

__device__ __forceinline__ int key_id(uint64_t k) {
  return (int)(0xFFFFFFFFu - (uint32_t)(k & 0xFFFFFFFFu));
}

constexpr int kCap = 128;  // survivors of the threshold a row can rank (2 per lane)

// LDS a selecting workgroup of NW waves needs (NW = 4, or 8 for one long
// row).  Row slot q of a pass is served by waves q * parts .. q * parts +
// parts - 1.
template <int NW>
struct SelectLds {
  uint64_t survivors[NW == 8 ? 1 : 4][kCap];  // keys at or above the row's threshold
  // list path, 4 waves: wave w's picks at [w * K1, w * K1 + K1) (8 waves put
  // their picks among the survivors instead)
  uint64_t finalists[NW == 8 ? 1 : 4 * kList];
  uint64_t bound[NW];  // per wave: its bound (K1-th largest score word << 32), or 0
  int32_t count[4];    // survivors per row slot
  int32_t row_sel[4][kMaxTopk];
};

// Batch slots (of kBatch) the wave needs for the candidates c0, c0 + stride,
// ... below `local`, for lane `lane` (lanes of a wave start at most 63
// apart, so lane 0's count covers every lane).
__device__ __forceinline__ int wave_slots(int c0, int lane, int stride, int local) {
  const int c0min = c0 - lane;
  if (local <= c0min) return 0;
  return min(kBatch, (local - c0min + stride - 1) / stride);
}

__device__ __forceinline__ uint64_t key_of(uint32_t ord, int c) {
  return ((uint64_t)ord << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)c);
}

// Orderable scores of a batch (ok, 0 past `local`: below every real key)
// folded into the lane's best key.  `nw`: the wave's slots.
__device__ __forceinline__ void key_batch(uint32_t (&ok)[kBatch], const float (&sv)[kBatch],
                                          uint64_t& best, int c0, int stride, int local,
                                          int nw) {
#pragma unroll
  for (int u = 0; u < kBatch; ++u) {
    if (u >= nw) break;  // wave-uniform
    const int c = c0 + u * stride;
    const uint32_t o = c < local ? orderable(sv[u]) : 0u;
    ok[u] = o;
    const uint64_t x = key_of(o, c);
    if (o != 0 && x > best) best = x;
  }
}

// Inserts a batch of candidates (ids c0, c0 + stride, ...; those >= local
// are skipped) into the lane's descending list of kList keys.
__device__ __forceinline__ void insert_batch(uint64_t (&list)[kList], const float (&sv)[kBatch],
                                             int c0, int stride, int local) {
#pragma unroll
  for (int u = 0; u < kBatch; ++u) {
    const int c = c0 + u * stride;
    if (c >= local) break;
    uint64_t x = make_key(sv[u], c);
    if (x > list[kList - 1]) {
#pragma unroll
      for (int j = 0; j < kList; ++j) {
        const uint64_t y = list[j];
        const bool gt = x > y;
        list[j] = gt ? x : y;
        x = gt ? y : x;
      }
    }
  }
}

// Loads the batch of candidates c0, c0 + stride, ... below `local` (0 past it).
__device__ __forceinline__ void load_batch(float (&sv)[kBatch], const float* srow, int c0,
                                           int stride, int local) {
#pragma unroll
  for (int u = 0; u < kBatch; ++u) {
    const int c = c0 + u * stride;
    sv[u] = c < local ? srow[c] : 0.f;
  }
}

// Lane j's value of a 64-bit key.
__device__ __forceinline__ uint64_t lane_key(uint64_t v, int j) {
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), j);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, j);
  return ((uint64_t)hi << 32) | lo;
}

// Selection (and, when page_table is given, the page table) for every row of
// request b.  Called by all threads of an NW-wave workgroup, of which the
// first NWS select (NWS = 8 only for single-row requests; the other waves
// only take part in the barriers); contains workgroup barriers.  page_row
// (LDS, T x topk x 8 ids): the rows' page ids are also left there, visible
// to the whole workgroup on return.
//
// Per row: every lane takes the best key among its candidates; each wave
// finds the K1-th largest score word of its lane maxima (K1 = topk - 1) bit
// by bit.  That word, as a key with zero low bits, has K1 real candidates
// at or above it, so no candidate below the largest of the row's wave
// bounds can be among the K1 best: only candidates reaching
// it survive (typically a few dozen), gathered in LDS and ranked by
// counting.  Rows with more than kCap survivors (a few lanes holding most of
// the best keys) take the list path instead: per-lane sorted lists of the
// K1 best keys, K1 wave-max pops per wave, and a merge-rank of the waves'
// picks.
template <int NWS, int NW = NWS>
__device__ __forceinline__ void select_request(int b, const float* __restrict__ scores,
                                            const int32_t* __restrict__ ctx_lens,
                                            const int32_t* __restrict__ block_table,
                                            int32_t* __restrict__ selected,
                                            int32_t* __restrict__ n_selected,
                                            int32_t* __restrict__ page_table, int T, int MAXB,
                                            int topk, SelectLds<NWS>& sh,
                                            int32_t* page_row = nullptr) {
  static_assert(NW >= NWS, "the selecting waves are the first NWS of the workgroup");
  const int lane = lane_id();
  const int wave = wave_id();
  const bool member = NW == NWS || wave < NWS;  // wave-uniform
  const int parts = NWS == 8 ? 8 : (T >= 4 ? 1 : (T == 1 ? 4 : (T == 2 ? 2 : 1)));
  const int rows_per_pass = NWS / parts;
  const int K1 = topk - 1;
  const int stride = parts * kWave;
  const int part = wave % parts;
  const int slot = wave / parts;
  const int cfirst = part * kWave + lane;
  auto& row_sel = sh.row_sel;

  for (int t0 = 0; t0 < T; t0 += rows_per_pass) {
    const int t = t0 + slot;
    // The first batch of scores is loaded together with the context length
    // (indices clamped into the row, rows into the request), so the two
    // round trips overlap; the empty asm pins the loads ahead of the branches
    // that use them.
    float sv[kBatch];
    if (member) {
      const float* srow = scores + (size_t)(b * T + min(t, T - 1)) * MAXB;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) sv[u] = srow[min(cfirst + u * stride, MAXB - 1)];
    } else {
#pragma unroll
      for (int u = 0; u < kBatch; ++u) sv[u] = 0.f;
    }
    int L = ctx_lens[b];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) asm volatile("" : "+v"(sv[u]));
    asm volatile("" : "+s"(L));
    // a context longer than its table row cannot send the candidates (and
    // the table lookups of the page build) past the row
    L = min(L, MAXB * 128);
    const bool active = member && t < T;
    const int r = b * T + t;
    const float* srow = scores + (size_t)r * MAXB;
    const int pos = L - T + t;
    const int local = pos >> 7;
    const bool take_all = local + 1 <= topk;
    // uniform over the row's waves
    const bool work = active && !take_all && K1 > 0;
    if (member && part == 0 && lane == 0) sh.count[slot] = 0;

    // lane maxima; the orderable scores of the first two batches (one with
    // 8 waves, which keeps the registers below 256) stay in registers
    constexpr bool kTwo = NWS == 4 && NW == 4;
    float sv2[kBatch];
    uint32_t ok0[kBatch], ok1[kBatch];
    const int c1 = cfirst + kBatch * stride;
    const int c2 = kTwo ? c1 + kBatch * stride : c1;  // first candidate re-read
    const int nw0 = wave_slots(cfirst, lane, stride, local);
    const int nw1 = wave_slots(c1, lane, stride, local);
    uint64_t lmax = 0;  // 0 ranks below every real key
    if (work) {
      if (kTwo && nw1 > 0) load_batch(sv2, srow, c1, stride, local);
      key_batch(ok0, sv, lmax, cfirst, stride, local, nw0);
      if (kTwo && nw1 > 0) key_batch(ok1, sv2, lmax, c1, stride, local, nw1);
      for (int c0 = c2; c0 - lane < local; c0 += kBatch * stride) {  // wave-uniform
        float sx[kBatch];
        uint32_t okx[kBatch];
        load_batch(sx, srow, c0, stride, local);
        key_batch(okx, sx, lmax, c0, stride, local, wave_slots(c0, lane, stride, local));
      }
    }
    // this wave's bound: the K1-th largest score word among its lane maxima
    // (0 when fewer than K1 lanes have a candidate), found bit by bit from
    // the top by counting the lanes at or above each trial value.  At least
    // K1 lane maxima, each a real candidate, reach (word << 32).
    uint64_t wbound = 0;
    if (work) {
      const uint32_t hi = (uint32_t)(lmax >> 32);
      uint32_t pre = 0;
#pragma unroll
      for (int bit = 31; bit >= 0; --bit) {
        const uint32_t trial = pre | (1u << bit);
        if (__popcll(__ballot(hi >= trial)) >= K1) pre = trial;
      }
      wbound = (uint64_t)pre << 32;
    }
    if (member && lane == 0) sh.bound[wave] = wbound;
    __syncthreads();

    // survivors: keys at or above the largest bound of the row's waves
    uint64_t bound = 0;
    for (int q = 0; q < parts && member; ++q) {
      const uint64_t x = sh.bound[slot * parts + q];
      bound = x > bound ? x : bound;
    }
    if (work) {
      // every key at or above the bound takes the next survivor slot by an
      // LDS atomic (the ranking below depends only on the keys, not on
      // their order)
      auto append = [&](const uint32_t (&ok)[kBatch], int c0, int nw) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          if (u >= nw) break;  // wave-uniform
          const uint64_t x = key_of(ok[u], c0 + u * stride);
          if (ok[u] != 0 && x >= bound) {
            const int i = atomicAdd(&sh.count[slot], 1);
            if (i < kCap) sh.survivors[slot][i] = x;
          }
        }
      };
      append(ok0, cfirst, nw0);
      if (kTwo) append(ok1, c1, nw1);
      for (int c0 = c2; c0 - lane < local; c0 += kBatch * stride) {  // wave-uniform
        float sx[kBatch];
        uint32_t okx[kBatch];
        uint64_t unused = 0;
        const int nw = wave_slots(c0, lane, stride, local);
        load_batch(sx, srow, c0, stride, local);
        key_batch(okx, sx, unused, c0, stride, local, nw);
        append(okx, c0, nw);
      }
    }
    __syncthreads();
    const int m = member ? sh.count[slot] : 0;
    const bool list_path = work && m > kCap;  // uniform over the row's waves

    if (list_path) {
      uint64_t list[kList];
#pragma unroll
      for (int j = 0; j < kList; ++j) list[j] = 0;
      for (int c0 = cfirst; c0 < local; c0 += kBatch * stride) {
        float sx[kBatch];
        load_batch(sx, srow, c0, stride, local);
        insert_batch(list, sx, c0, stride, local);
      }
      // this wave's K1 best keys, best first; 0 once its lists run dry
      uint64_t* picks = (NWS == 8 ? sh.survivors[slot] : sh.finalists) + wave * K1;
      for (int k = 0; k < K1; ++k) {
        const uint64_t best = wave_max_u64(list[0]);
        if (best == 0) {  // wave-uniform
          for (int e = lane; e < K1 - k; e += kWave) picks[k + e] = 0;
          break;
        }
        if (lane == 0) picks[k] = best;
        if (list[0] == best) {
#pragma unroll
          for (int j = 0; j < kList - 1; ++j) list[j] = list[j + 1];
          list[kList - 1] = 0;
        }
      }
    }
    __syncthreads();

    // 8 waves (one row): every wave ranks 16 of the (up to kCap) entries by
    // counting, each lane against a quarter of the entries, instead of one
    // wave ranking them all (the entries are the survivors, or on the list
    // path the waves' picks, zeros ranking below every key).
    if constexpr (NWS == 8) {
      if (work) {
        const int me = list_path ? parts * K1 : m;
        const uint64_t* sv_ = sh.survivors[slot];
        const int i = 16 * wave + (lane & 15);
        const int quarter = lane >> 4;
        const uint64_t e = i < me ? sv_[i] : 0;
        int cnt = 0;
        // 8 independent reads per step (kCap = 128 entries: at most 4 steps)
        for (int j0 = quarter; j0 < me; j0 += 32) {
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const int j = j0 + 4 * q;
            const uint64_t x = sv_[min(j, kCap - 1)];
            cnt += (j < me && x > e) ? 1 : 0;
          }
        }
        cnt += __shfl_xor(cnt, 16);
        cnt += __shfl_xor(cnt, 32);
        if (quarter == 0 && i < me && e != 0 && cnt < K1) row_sel[slot][cnt] = key_id(e);
      }
      __syncthreads();
    }

    if (active && part == 0) {
      int n = 0;
      if (take_all) {
        n = local + 1;
        for (int k = lane; k < n; k += kWave) row_sel[wave][k] = k;
      } else if (K1 == 0) {
        if (lane == 0) row_sel[wave][0] = local;
        n = 1;
      } else {
        // the K1 best keys go to row_sel[wave][rank] (keys are unique, so
        // ranks 0 .. K1 - 1 each have exactly one owner); with 8 waves that
        // happened above
        if (NWS == 8) {
        } else if (!list_path) {
          // rank by counting among the survivors
          const int me = m;
          uint64_t* sv_ = sh.survivors[slot];
          const uint64_t e0 = lane < me ? sv_[lane] : 0;
          const uint64_t e1 = lane + kWave < me ? sv_[lane + kWave] : 0;
          // zeros up to a multiple of 8 (they rank below every key), then
          // 8 keys per step
          if (lane < 8 && me + lane < kCap) sv_[me + lane] = 0;
          __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
          __builtin_amdgcn_wave_barrier();
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
          int r0 = 0, r1 = 0;
          for (int j = 0; j < me; j += 8) {
#pragma unroll
            for (int q = 0; q < 8; ++q) {
              const uint64_t x = sv_[j + q];
              r0 += x > e0 ? 1 : 0;
              r1 += x > e1 ? 1 : 0;
            }
          }
          if (lane < me && r0 < K1) row_sel[wave][r0] = key_id(e0);
          if (lane + kWave < me && r1 < K1) row_sel[wave][r1] = key_id(e1);
        } else {
          // merge-rank of the waves' picks: each wave's list is sorted best
          // first (zeros last) and keys are unique, so a pick's rank is its
          // index plus, per other list, the count of better keys there (a
          // binary search)
          const int mf = parts * K1;
          const uint64_t* fin = sh.finalists + wave * K1;
          const uint64_t mine = lane < mf ? fin[lane] : 0;
          const int own = lane < mf ? lane / K1 : 0;
          int rank = lane - own * K1;
          for (int w = 0; w < parts; ++w) {  // wave-uniform
            if (w == own) continue;
            const uint64_t* list = fin + w * K1;
            int cnt = 0;
#pragma unroll
            for (int step = 8; step >= 1; step >>= 1)
              if (cnt + step <= K1 && list[cnt + step - 1] > mine) cnt += step;
            rank += cnt;
          }
          if (lane < mf && rank < K1 && mine != 0) row_sel[wave][rank] = key_id(mine);
        }
        // order the K1 winners by id: lane k places the k-th ranked one,
        // its position counted from the other winners' ids in registers
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const int id = lane < K1 ? row_sel[wave][lane] : INT32_MAX;
        int posn = 0;
#pragma unroll
        for (int e = 0; e < kList; ++e) {
          const int o = __builtin_amdgcn_readlane(id, e);
          posn += o < id ? 1 : 0;
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (lane < K1) row_sel[wave][posn] = id;
        if (lane == 0) row_sel[wave][K1] = local;
        n = topk;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (selected)
        for (int k = lane; k < topk; k += kWave)
          selected[(size_t)r * topk + k] = k < n ? row_sel[wave][k] : -1;
      if (lane == 0 && n_selected) n_selected[r] = n;
      if (page_table || page_row) {
        // one table lookup per kept block (lane k), then page entry e takes
        // block e / 8's id from that lane (topk <= 16: at most two entries
        // per lane)
        static_assert(kMaxTopk * 8 <= 2 * kWave, "two page entries per lane");
        const int pt = topk * 8;
        const int phys = lane < n ? block_table[(size_t)b * MAXB + row_sel[wave][lane]] : -1;
        const int p0 = __shfl(phys, lane >> 3);
        const int p1 = __shfl(phys, (lane + kWave) >> 3);
        for (int e = lane; e < pt; e += kWave) {
          const int k = e >> 3;
          const int v = k < n ? (e < kWave ? p0 : p1) * 8 + (e & 7) : -1;
          if (page_table) page_table[(size_t)r * pt + e] = v;
          if (page_row) page_row[(size_t)t * pt + e] = v;
        }
      }
    }
    __syncthreads();
  }
}

}  // namespace msa
