// paged_decode.hip - entry points of the decode split and reduce kernels
// (paged_decode.hpp): dispatch on the head dimension to the instantiation
// units paged_decode_d{64,128,256}.hip, and the partition merge that the
// chunked prefill shares.
#include "paged_decode.hpp"

namespace kvfp8 {

hipError_t launch_paged_decode_hd64(const DecodeParams& p, int fmt, int num_seqs, bool fused,
                                    int slots, int tile_pages, int mode, hipStream_t stream,
                                    hipEvent_t ev_before, hipEvent_t ev_after);
hipError_t launch_paged_decode_hd128(const DecodeParams& p, int fmt, int num_seqs, bool fused,
                                     int slots, int tile_pages, int mode, hipStream_t stream,
                                     hipEvent_t ev_before, hipEvent_t ev_after);
hipError_t launch_paged_decode_hd256(const DecodeParams& p, int fmt, int num_seqs, bool fused,
                                     int slots, int tile_pages, int mode, hipStream_t stream,
                                     hipEvent_t ev_before, hipEvent_t ev_after);

hipError_t launch_partition_merge(const DecodeParams& p, int head_dim, int rows,
                                  hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  switch (head_dim) {
    case 64: launch_reduce<64>(p, rows, stream); break;
    case 128: launch_reduce<128>(p, rows, stream); break;
    case 256: launch_reduce<256>(p, rows, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_paged_decode(const DecodeParams& p, int head_dim, int fmt, int num_seqs,
                               bool fused, int slots, int tile_pages, bool att8, bool dyn,
                               hipStream_t stream, hipEvent_t ev_before, hipEvent_t ev_after) {
  if (att8 && dyn) return hipErrorInvalidValue;
  const int mode = att8 ? kModeFp8 : dyn ? kModeDyn : kModeBf16;
  switch (head_dim) {
    case 64:
      return launch_paged_decode_hd64(p, fmt, num_seqs, fused, slots, tile_pages, mode, stream,
                                      ev_before, ev_after);
    case 128:
      return launch_paged_decode_hd128(p, fmt, num_seqs, fused, slots, tile_pages, mode, stream,
                                       ev_before, ev_after);
    case 256:
      return launch_paged_decode_hd256(p, fmt, num_seqs, fused, slots, tile_pages, mode, stream,
                                       ev_before, ev_after);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace kvfp8
