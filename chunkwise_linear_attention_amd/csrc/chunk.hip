// Chunkwise linear attention kernels (placeholder until the MFMA kernels land).
#include "internal.h"

namespace cla {

ChunkPlan plan_chunk(int64_t B, int64_t H, int64_t T, int64_t DK, int64_t DV) {
  (void)B; (void)H; (void)T; (void)DK; (void)DV;
  return ChunkPlan{};
}

hipError_t launch_chunk_fwd(const uint16_t *, const uint16_t *, const uint16_t *,
                            const float *, const float *, uint16_t *, float *,
                            int64_t, int64_t, int64_t, int64_t, int64_t,
                            const ChunkPlan &, void *, hipStream_t) {
  return hipErrorNotSupported;
}

hipError_t launch_chunk_bwd(const uint16_t *, const uint16_t *, const uint16_t *,
                            const float *, const float *, const uint16_t *,
                            const float *, uint16_t *, uint16_t *, uint16_t *,
                            float *, float *, int64_t, int64_t, int64_t, int64_t,
                            int64_t, const ChunkPlan &, void *, hipStream_t) {
  return hipErrorNotSupported;
}

}  // namespace cla
