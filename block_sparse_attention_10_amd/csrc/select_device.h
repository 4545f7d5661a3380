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
// T < 4).  Every lane streams its candidates in ascending id order into a
// register-resident sorted list of the topk - 1 best 64-bit keys (orderable
// score << 32 | ~id, so a larger key is a better block and equal scores
// favour the lower id).  Each wave then pops its topk - 1 best keys by
// repeated wave maxima (DPP reductions, no LDS traffic), the waves of a row
// meet in LDS, and one wave ranks the union (at most 60 finalists, one per
// lane), sorts the winners by id and writes the row's selection and page
// table.
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

// LDS a selecting workgroup needs.
struct SelectLds {
  uint64_t finalists[4 * kList];  // wave w's picks at [w * K1, w * K1 + K1)
  int32_t row_sel[4][kMaxTopk];
};

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

// Selection (and, when page_table is given, the page table) for every row of
// request b.  Called by all 256 threads of a 4-wave workgroup; contains
// workgroup barriers.
__device__ __forceinline__ void select_request(int b, const float* __restrict__ scores,
                                            const int32_t* __restrict__ ctx_lens,
                                            const int32_t* __restrict__ block_table,
                                            int32_t* __restrict__ selected,
                                            int32_t* __restrict__ n_selected,
                                            int32_t* __restrict__ page_table, int T, int MAXB,
                                            int topk, SelectLds& sh) {
  uint64_t* finalists = sh.finalists;
  auto& row_sel = sh.row_sel;
  const int lane = lane_id();
  const int wave = wave_id();
  const int parts = T >= 4 ? 1 : (T == 1 ? 4 : (T == 2 ? 2 : 1));
  const int rows_per_pass = 4 / parts;
  const int K1 = topk - 1;
  const int stride = parts * kWave;
  const int part = wave % parts;
  const int cfirst = part * kWave + lane;

  for (int t0 = 0; t0 < T; t0 += rows_per_pass) {
    const int t = t0 + wave / parts;
    // The first batch of scores is loaded together with the context length
    // (indices clamped into the row, rows into the request), so the two
    // round trips overlap; the empty asm pins the loads ahead of the branches
    // that use them.
    float sv[kBatch];
    {
      const float* srow = scores + (size_t)(b * T + min(t, T - 1)) * MAXB;
#pragma unroll
      for (int u = 0; u < kBatch; ++u) sv[u] = srow[min(cfirst + u * stride, MAXB - 1)];
    }
    int L = ctx_lens[b];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) asm volatile("" : "+v"(sv[u]));
    asm volatile("" : "+s"(L));
    const bool active = t < T;
    const int r = b * T + t;
    const float* srow = scores + (size_t)r * MAXB;
    const int pos = L - T + t;
    const int local = pos >> 7;
    const bool take_all = local + 1 <= topk;

    if (active && !take_all && K1 > 0) {
      uint64_t list[kList];
#pragma unroll
      for (int j = 0; j < kList; ++j) list[j] = 0;  // 0 ranks below every real key
      insert_batch(list, sv, cfirst, stride, local);
      for (int c0 = cfirst + kBatch * stride; c0 < local; c0 += kBatch * stride) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int c = c0 + u * stride;
          sv[u] = c < local ? srow[c] : 0.f;
        }
        insert_batch(list, sv, c0, stride, local);
      }
      // this wave's K1 best keys, best first; 0 once its lists run dry
      for (int k = 0; k < K1; ++k) {
        const uint64_t best = wave_max_u64(list[0]);
        if (best == 0) {  // wave-uniform
          for (int e = lane; e < K1 - k; e += kWave) finalists[wave * K1 + k + e] = 0;
          break;
        }
        if (lane == 0) finalists[wave * K1 + k] = best;
        if (list[0] == best) {
#pragma unroll
          for (int j = 0; j < kList - 1; ++j) list[j] = list[j + 1];
          list[kList - 1] = 0;
        }
      }
    }
    __syncthreads();

    if (active && part == 0) {
      int n = 0;
      if (take_all) {
        n = local + 1;
        for (int k = lane; k < n; k += kWave) row_sel[wave][k] = k;
      } else if (K1 == 0) {
        if (lane == 0) row_sel[wave][0] = local;
        n = 1;
      } else {
        // rank the union of this row's per-wave picks (waves wave ..
        // wave + parts - 1, stored contiguously).  Each wave's list is sorted
        // best first (pop order, zeros last) and keys are unique, so a pick's
        // rank is its index plus, per other list, the count of better keys
        // there (a binary search).
        const int m = parts * K1;
        const uint64_t* fin = finalists + wave * K1;
        const uint64_t mine = lane < m ? fin[lane] : 0;
        const int own = lane < m ? lane / K1 : 0;
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
        const bool win = lane < m && rank < K1 && mine != 0;
        const int id = key_id(mine);
        // position among the winners by ascending id
        __builtin_amdgcn_wave_barrier();
        if (win) row_sel[wave][rank] = id;
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        int posn = 0;
#pragma unroll
        for (int e = 0; e < kList; ++e) {
          const int o = e < K1 ? row_sel[wave][e] : INT32_MAX;
          posn += o < id ? 1 : 0;
        }
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (win) row_sel[wave][posn] = id;
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
      if (page_table) {
        const int pt = topk * 8;
        for (int e = lane; e < pt; e += kWave) {
          const int k = e >> 3;
          int v = -1;
          if (k < n) v = block_table[(size_t)b * MAXB + row_sel[wave][k]] * 8 + (e & 7);
          page_table[(size_t)r * pt + e] = v;
        }
      }
    }
    __syncthreads();
  }
}

}  // namespace msa
