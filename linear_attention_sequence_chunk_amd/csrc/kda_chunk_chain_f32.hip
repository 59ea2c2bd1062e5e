// kda_chunk_chain_f32.hip -- stage 2 instantiations for f32 inputs.
#include "kda_chunk_chain.h"

namespace kda {

hipError_t run_chunk_chain_f32(const ChunkArgs& a) {
    return a.out_bf16 ? chain_dims<float, bf16>(a) : chain_dims<float, float>(a);
}

}  // namespace kda
