// paged_decode_d256.hip - the decode split and reduce kernels (paged_decode.hpp)
// instantiated for head dimension 256.
#include "paged_decode.hpp"

namespace kvfp8 {

hipError_t launch_paged_decode_hd256(const DecodeParams& p, int fmt, int num_seqs, bool fused,
                                   int slots, int tile_pages, int mode, hipStream_t stream,
                                   hipEvent_t ev_before, hipEvent_t ev_after) {
  return launch_dim<256>(p, fmt, num_seqs, fused, slots, tile_pages, mode, stream, ev_before,
                        ev_after);
}

}  // namespace kvfp8
