// Overflow-row set of the gate kernels (both tile shapes).
//
// A row overflows when one of its (row, tile) counts exceeds C; its rows go
// to the dense fallback (rows that do not fit the sparse block fall back to a
// dense buffer: Telegram post on TwELL at tgviewer.app, part "Обучение";
// Tencent Cloud article, section 3). The set is built
// with device-scope atomics in the caller's control block, which is zero
// before every call and left zero after it:
//   word 0 (64-bit): low half = rows appended so far, high half = workgroups
//                    finished;
//   word 2: spill records taken (training gate only);
//   then one dedup flag per row.
// Appends and arrivals use the one 64-bit word, so the workgroup that arrives
// last learns from its own arrival both that it is last and how many rows were
// appended (every append precedes its workgroup's arrival: the appending wave
// fences before the workgroup barrier). With no overflow rows it then only
// stores n_ovf and clears the word: one device-scope round trip in all.
#pragma once

#include "twell_device.hpp"
#include "twell_internal.hpp"

namespace twell {

// Appends `row` unless it is in the set already; returns 1 if this call added it.
__device__ __forceinline__ int overflow_append(const GateArgs& a, int row) {
  uint32_t* flags = a.ctrl + kCtrlBytes / 4;
  if (atomicExch(&flags[row], 1u) != 0u) return 0;
  uint64_t* word = reinterpret_cast<uint64_t*>(a.ctrl);
  const uint32_t pos = static_cast<uint32_t>(
      __hip_atomic_fetch_add(word, uint64_t{1}, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  // pos < M whenever the control block started zeroed, as the API requires
  if (pos < static_cast<uint32_t>(a.M))
    __hip_atomic_store(&a.ovf_rows[pos], row, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return 1;
}

// Called by every thread of every workgroup once its appends are issued.
// `appended`: this thread added a row. `s_flag`: one int of LDS that no wave
// reads or writes any more.
__device__ __forceinline__ void overflow_finalize(const GateArgs& a, int appended, int* s_flag) {
  // Only waves that appended rows have list entries to release; the barriers
  // carry no fence, so other waves need not wait for their packing stores.
  if (__ballot(appended) != 0) __threadfence();
  raw_barrier();
  uint64_t* word = reinterpret_cast<uint64_t*>(a.ctrl);
  if (threadIdx.x == 0) {
    const uint64_t old =
        __hip_atomic_fetch_add(word, uint64_t{1} << 32, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = static_cast<uint32_t>(old >> 32) == gridDim.x - 1u;
    const uint32_t n = min(static_cast<uint32_t>(old), static_cast<uint32_t>(a.M));
    *s_flag = last ? static_cast<int>(n) + 1 : 0;  // 0: not last, else 1 + rows
  }
  waitcnt<63, 0>();  // the flag store has reached LDS
  raw_barrier();
  const int f = *s_flag;
  if (f == 0) return;
  const uint32_t n = static_cast<uint32_t>(f - 1);
  if (n > 0) {
    __threadfence();  // acquire the other workgroups' list entries
    uint32_t* flags = a.ctrl + kCtrlBytes / 4;
    for (uint32_t i = threadIdx.x; i < n; i += blockDim.x) {
      const int r = __hip_atomic_load(&a.ovf_rows[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (r >= 0 && r < a.M) __hip_atomic_store(&flags[r], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  if (threadIdx.x == 0) {
    *a.n_ovf = static_cast<int32_t>(n);
    if (a.rec_n != nullptr) {  // spill records: publish the count, clear the counter
      if (n == 0) __threadfence();  // (no fence was taken above)
      uint32_t* rc = a.ctrl + 2;
      *a.rec_n = static_cast<int32_t>(__hip_atomic_load(rc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      __hip_atomic_store(rc, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __hip_atomic_store(word, uint64_t{0}, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace twell
