// kda_chunk_chain_bf16.hip -- stage 2 instantiations for bf16 inputs.
#include "kda_chunk_chain.h"

namespace kda {

hipError_t run_chunk_chain_bf16(const ChunkArgs& a) {
    return a.out_bf16 ? chain_dims<bf16, bf16>(a) : chain_dims<bf16, float>(a);
}

}  // namespace kda
