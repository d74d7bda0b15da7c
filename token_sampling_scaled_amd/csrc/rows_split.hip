// Split-row kernel for rows sampled without a filter (every row of a call on
// the no-filter route): the Gumbel-max draw needs Philox noise for every entry
// of the row, so the work is VALU-bound and a row is spread over S workgroups
// of 256 threads, each taking a contiguous run of 4-entry groups (one Philox
// block per group).  Each workgroup leaves a partial result -- its perturbed
// argmax and the log-sum-exp of its entries as (max, sum) -- in the handle's
// workspace; the last workgroup of the row to finish (a per-row counter taken
// with a device-scope atomic) merges the S partials in a fixed order, so the
// result does not depend on which workgroup finishes last, and resets the
// counter for the next call.
//
// Per row (no-filter reading of the processed distribution): P = every entry
// above -inf (NaN reads as -inf); id = argmax_P (x/T + g), lowest index on
// ties; lp = x_id/T - logsumexp_P(x/T).  Rows with T < 1e-5 take the first
// maximum with lp = 0; a row with no entry above -inf gives id -1, lp NaN.
#include "split_common.hpp"

namespace tss {

namespace {

using namespace split;

// PT: 4-entry groups per thread; S workgroups per row (gridDim.x = n * S,
// part-major: workgroup b takes row b % n, part b / n).  RAW: no noise and no
// temperature; the merge writes the log-softmax of the raw row at
// token_ids[r] (out_lp[r]) instead of a sample.
template <typename T, bool VEC, int PT, bool RAW>
__global__ __launch_bounds__(kSplitBlock) void rows_split_none_kernel(RowArgs a, int32_t S) {
  using E = SplitElem<T>;
  using K = typename E::Key;
  __shared__ Best sbest[kSplitWaves];
  __shared__ Lse slse[kSplitWaves];
  __shared__ uint32_t sticket;

  const int r = (int)(blockIdx.x % (uint32_t)a.n);
  const int part = (int)(blockIdx.x / (uint32_t)a.n);
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  const int64_t src = a.gather ? (int64_t)a.gather[r] : (int64_t)r;
  const int64_t q = a.req_map ? (int64_t)a.req_map[r] : (int64_t)r;
  const T* row = reinterpret_cast<const T*>(a.logits) + src * a.row_stride;
  const int64_t v = a.vocab;
  const int32_t groups = (int32_t)((v + 3) >> 2);
  const int32_t per_part = (groups + S - 1) / S;
  const int32_t g_begin = part * per_part;
  const int32_t g_end = g_begin + per_part < groups ? g_begin + per_part : groups;
  const float temp = RAW ? 1.0f : a.temperature[q];
  const uint64_t seed = RAW ? 0ull : a.seed[q];
  const bool greedy = !RAW && !(temp >= 1e-5f);
  // base-2 units: s2 = x * log2(e) / T.  The Gumbel race is run as
  // argmax (s2 - log2(-log2 u)), which is argmax (x/T - ln(-ln u)) scaled by
  // log2(e) and shifted by a constant; the log-sum-exp uses exp2.
  const float scale2 = greedy ? 1.0f : 1.4426950408889634f / temp;

  // ---- load this thread's groups, all loads in flight at once.  With VEC
  // (vocab a multiple of 4, aligned rows) every load is unconditional: a slot
  // past this part re-reads the part's last group and is masked below.
  uint32_t raw[PT][4];
  if (VEC) {
    typename E::Packed pk[PT];
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int32_t g = g_begin + tid + i * kSplitBlock;
      pk[i] = E::load_packed(row, (int64_t)(g < g_end ? g : g_end - 1) * 4);
    }
    __builtin_amdgcn_sched_barrier(0);   // keep every load ahead of the first use
#pragma unroll
    for (int i = 0; i < PT; ++i) E::unpack(pk[i], raw[i]);
  } else {
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int32_t g = g_begin + tid + i * kSplitBlock;
      if (g < g_end) {
        E::load4(row, (int64_t)g * 4, v, raw[i]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) raw[i][e] = E::kNegInfRaw;
      }
    }
  }

  Best best{0u, 0x7FFFFFFF, 0.0f};
  Lse lse{-__builtin_inff(), 0.0f};
  if (greedy) {
    // first maximum of the order key (NaN as -inf, -0 as +0), lp = 0
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const int32_t g = g_begin + tid + i * kSplitBlock;
      if (g >= g_end) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t key = K::from_bits(raw[i][e]);
        const int32_t j = g * 4 + e;
        if (key > K::kNegInf && key > best.o) best = Best{key, j, 0.0f};   // j rises
      }
    }
  } else {
    // scaled logits (NaN as -inf; -inf entries drop out of the sum and can
    // never win) and their maximum, for the log-sum-exp
    float sv[PT][4];
    float mloc = -__builtin_inff();
#pragma unroll
    for (int i = 0; i < PT; ++i) {
      const bool in = g_begin + tid + i * kSplitBlock < g_end;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float x = E::value(raw[i][e]);
        sv[i][e] = (in && x == x) ? x * scale2 : -__builtin_inff();
        mloc = fmaxf(mloc, sv[i][e]);
      }
    }
    float sum = 0.0f;
    if constexpr (RAW) {
#pragma unroll
      for (int i = 0; i < PT; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) sum += __builtin_amdgcn_exp2f(sv[i][e] - mloc);   // 0 for -inf
    }
    const uint64_t off = RAW ? 0ull : noise_offset(a, q);
    const NoiseStream ns{(uint32_t)seed, (uint32_t)(seed >> 32), (uint32_t)r,
                         (uint32_t)off, (uint32_t)(off >> 32)};
    float bz = -__builtin_inff();
    int32_t bj = 0x7FFFFFFF;
    float bs = 0.0f;
#pragma unroll
    for (int i = 0; i < (RAW ? 0 : PT); ++i) {
      const int32_t g = g_begin + tid + i * kSplitBlock;
      const Philox4 w = ns.block((uint32_t)g);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float s = sv[i][e];
        sum += __builtin_amdgcn_exp2f(s - mloc);       // 0 for -inf
        const float z = s + gumbel2_from_word(w.v[e]);
        if (z > bz) {                                  // j rises: first of equals stays
          bz = z;
          bj = g * 4 + e;
          bs = s;
        }
      }
    }
    if (mloc == -__builtin_inff()) sum = 0.0f;
    if (bz > -__builtin_inff()) best = Best{order_of(bz), bj, bs};
    lse = Lse{mloc, sum};
  }

  // ---- workgroup reduction, then this part's partial result
  best = wave_best(best);
  lse = wave_lse(lse);
  if (lane == 0) {
    sbest[wid] = best;
    slse[wid] = lse;
  }
  __syncthreads();
  SplitPartial* parts = reinterpret_cast<SplitPartial*>(a.split_partials) + (int64_t)r * S;
  if (tid == 0) {
    Best b = sbest[0];
    Lse l = slse[0];
#pragma unroll
    for (int w = 1; w < kSplitWaves; ++w) {
      if (beats(sbest[w].o, sbest[w].j, b.o, b.j)) b = sbest[w];
      l = lse_merge(l, slse[w]);
    }
    SplitPartial* p = parts + part;
    store_agent(&p->o, b.o);
    store_agent(&p->j, b.j);
    store_agent(&p->s, b.s);
    store_agent(&p->m, l.m);
    store_agent(&p->sum, l.sum);
    // The partial goes out as device-coherent (sc1) stores, which write
    // through to the coherence point; once they are acknowledged (vmcnt 0)
    // the counter is bumped.  The workgroup that takes the last ticket has
    // seen every other bump, so every partial has landed, and it reads them
    // back with device-coherent loads.  (A release / acquire pair would also
    // write back and invalidate whole L2 caches on every workgroup.)
    // Basis: the GFX942/GFX950 memory model of the LLVM AMDGPU backend
    // (AMDGPUUsage, "Memory Model GFX942"): agent-scope atomic stores and
    // loads are sc1 accesses that reach the coherence point past the per-XCD
    // L2, and an agent-scope release is an L2 write-back plus s_waitcnt
    // vmcnt(0).  The write-back only matters for ordinary stores; the
    // partial has none, so the wait alone orders its stores before the
    // ticket.
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
    sticket = __hip_atomic_fetch_add(a.split_counter + r, 1u, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (sticket != (uint32_t)(S - 1) || wid != 0) return;

  // ---- last workgroup of the row: merge the S partials in part order
  Best b{0u, 0x7FFFFFFF, 0.0f};
  Lse l{-__builtin_inff(), 0.0f};
  for (int p0 = 0; p0 < S; p0 += kWave) {
    Best bb{0u, 0x7FFFFFFF, 0.0f};
    Lse ll{-__builtin_inff(), 0.0f};
    if (p0 + lane < S) {
      const SplitPartial* p = parts + p0 + lane;
      bb = Best{load_agent_u(&p->o), load_agent_i(&p->j), load_agent_f(&p->s)};
      ll = Lse{load_agent_f(&p->m), load_agent_f(&p->sum)};
    }
    bb = wave_best(bb);
    ll = wave_lse(ll);
    if (beats(bb.o, bb.j, b.o, b.j)) b = bb;
    l = lse_merge(l, ll);
  }
  if (RAW && lane == 0) {
    // log-softmax of the raw row at the given id: NaN for an id outside the
    // row or a row with no finite entry, -inf at a NaN or -inf entry
    const int64_t j = a.token_ids[r];
    float out = __builtin_nanf("");
    if (j >= 0 && j < v && l.m > -__builtin_inff()) {
      const float x = E::value(E::raw_at(row, j));
      out = x == x ? (x * 1.4426950408889634f - l.m - __builtin_amdgcn_logf(l.sum)) *
                         0.69314718055994531f
                   : -__builtin_inff();
    }
    a.out_lp[r] = out;
    __hip_atomic_store(a.split_counter + r, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else if (lane == 0) {
    if (b.j == 0x7FFFFFFF) {
      a.out_ids[r] = -1;
      if (a.out_lp) a.out_lp[r] = __builtin_nanf("");
    } else {
      a.out_ids[r] = b.j;
      if (a.out_lp)
        a.out_lp[r] = greedy ? 0.0f : (b.s - l.m - __builtin_amdgcn_logf(l.sum)) * 0.69314718055994531f;
    }
    __hip_atomic_store(a.split_counter + r, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

template <typename T, bool VEC, bool RAW>
hipError_t launch_pt(const RowArgs& a, int32_t S, int pt, hipStream_t stream) {
  const dim3 grid((uint32_t)a.n * (uint32_t)S), block(kSplitBlock);
  switch (pt) {
    case 4:
      hipLaunchKernelGGL((rows_split_none_kernel<T, VEC, 4, RAW>), grid, block, 0, stream, a, S);
      break;
    case 8:
      hipLaunchKernelGGL((rows_split_none_kernel<T, VEC, 8, RAW>), grid, block, 0, stream, a, S);
      break;
    default:
      hipLaunchKernelGGL((rows_split_none_kernel<T, VEC, 16, RAW>), grid, block, 0, stream, a, S);
      break;
  }
  return hipGetLastError();
}

template <bool RAW>
hipError_t launch_split(const RowArgs& a, DType dtype, hipStream_t stream) {
  if (a.n <= 0) return hipSuccess;
  const int64_t groups = (a.vocab + 3) >> 2;
  // with noise (VALU-bound) about 4 groups (16 entries) per thread; without
  // (HBM-bound) about 16, so fewer workgroups merge; at most kMaxSplit parts
  constexpr int kPer = RAW ? 16 : 4;
  int64_t s = (groups + kPer * kSplitBlock - 1) / (kPer * kSplitBlock);
  if (s > kMaxSplit) s = kMaxSplit;
  if (s < 1) s = 1;
  const int64_t per_part = (groups + s - 1) / s;
  const int64_t per_thread = (per_part + kSplitBlock - 1) / kSplitBlock;
  const int pt = per_thread <= 4 ? 4 : per_thread <= 8 ? 8 : 16;
  const uintptr_t base = reinterpret_cast<uintptr_t>(a.logits);
  if (dtype == kF32) {
    const bool vec = (base % 16) == 0 && (a.row_stride % 4) == 0 && (a.vocab % 4) == 0;
    return vec ? launch_pt<float, true, RAW>(a, (int32_t)s, pt, stream)
               : launch_pt<float, false, RAW>(a, (int32_t)s, pt, stream);
  }
  const bool vec = (base % 8) == 0 && (a.row_stride % 4) == 0 && (a.vocab % 4) == 0;
  return vec ? launch_pt<uint16_t, true, RAW>(a, (int32_t)s, pt, stream)
             : launch_pt<uint16_t, false, RAW>(a, (int32_t)s, pt, stream);
}

}  // namespace

bool split_none_supported(const RowArgs& a) {
  const int64_t groups = (a.vocab + 3) >> 2;
  return a.split_counter != nullptr && a.split_partials != nullptr &&
         groups <= (int64_t)kMaxSplit * kSplitBlock * 16 &&
         (int64_t)a.n * kMaxSplit < 0x7FFFFFFF;
}

hipError_t launch_rows_split_none(const RowArgs& a, DType dtype, hipStream_t stream) {
  return launch_split<false>(a, dtype, stream);
}

hipError_t launch_rows_raw_log_prob_at(const RowArgs& a, DType dtype, hipStream_t stream) {
  return launch_split<true>(a, dtype, stream);
}

}  // namespace tss
