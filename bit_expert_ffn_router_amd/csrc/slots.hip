// Resident-expert slot table edits.  The pages keep the most used experts
// resident on the GPU and swap them while serving ([AF] "个人开发者用 AI 十天
// 写出 Strata 引擎…", section "命中率七成，代价是答案会变"; [JD]
// "5070ti16g单卡跑qwen 3.8 flash next …", section "为什么从 18t/s 变成
// 60-90t/s").  The host validates each update against its mirror of the
// table; these kernels apply the already-validated map edits on the stream.
#include "kernels.hpp"

namespace moe {

struct SlotEditBatch {
  SlotEdit e[kSlotEditsPerLaunch];
};

// One thread per edit.  Phase 0 evicts: the slot's previous occupant stops
// being resident.  Phase 1 installs: the slot takes its new expert (or
// becomes empty).  The host runs phase 0 over every batch of a call before
// phase 1 over any, so an expert moved from a slot that a later batch edits
// keeps its new slot.
__global__ void slot_edit_kernel(int32_t* slot_of, int32_t* expert_of_slot, SlotEditBatch b,
                                 int n, int phase) {
  const int i = threadIdx.x;
  if (i >= n) return;
  if (phase == 0) {
    if (b.e[i].old_expert >= 0) slot_of[b.e[i].old_expert] = -1;
  } else {
    expert_of_slot[b.e[i].slot] = b.e[i].expert;
    if (b.e[i].expert >= 0) slot_of[b.e[i].expert] = b.e[i].slot;
  }
}

// Halve every usage count (the decay step of the slot policy's statistics).
__global__ void counts_halve_kernel(uint32_t* counts, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) counts[i] >>= 1;
}

hipError_t launch_counts_halve(uint32_t* counts, int n, hipStream_t st) {
  counts_halve_kernel<<<(n + 255) / 256, 256, 0, st>>>(counts, n);
  return hipGetLastError();
}

__global__ void slot_init_kernel(int32_t* slot_of, int E, int32_t* expert_of_slot, int S) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < E) slot_of[i] = -1;
  if (i < S) expert_of_slot[i] = -1;
}

hipError_t launch_slot_edits(int32_t* slot_of, int32_t* expert_of_slot, const SlotEdit* edits,
                             int n, hipStream_t st) {
  for (int phase = 0; phase < 2; ++phase)
    for (int i0 = 0; i0 < n; i0 += kSlotEditsPerLaunch) {
      const int m = n - i0 < kSlotEditsPerLaunch ? n - i0 : kSlotEditsPerLaunch;
      SlotEditBatch b;
      for (int i = 0; i < m; ++i) b.e[i] = edits[i0 + i];
      slot_edit_kernel<<<1, kSlotEditsPerLaunch, 0, st>>>(slot_of, expert_of_slot, b, m, phase);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  return hipSuccess;
}

hipError_t launch_slot_init(int32_t* slot_of, int E, int32_t* expert_of_slot, int S,
                            hipStream_t st) {
  const int m = E > S ? E : S;
  slot_init_kernel<<<(m + 255) / 256, 256, 0, st>>>(slot_of, E, expert_of_slot, S);
  return hipGetLastError();
}

}  // namespace moe
