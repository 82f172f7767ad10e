// Launch functions for the host-only sanitizer build of the C-ABI layer
// (mosaic_bsa_api.cpp built by g++ with -fsanitize=address,undefined).  The
// ABI tests only pass arguments that validation rejects, so none of these
// may ever run: each one records that it was reached and reports a HIP
// error, which the tests see as MOSAIC_ERR_HIP instead of the status they
// expect.
#include "bsa_launch.h"

namespace mosaic {

extern "C" {
int mosaic_test_stub_calls = 0;
}

namespace {
hipError_t reached() {
  ++mosaic_test_stub_calls;
  return hipErrorInvalidValue;
}
}  // namespace

hipError_t launch_pool(const uint16_t*, const uint16_t*, const uint16_t*, double*, double*, float*, long long, int,
                       int, int, hipStream_t, float*, uint16_t*, float*) {
  return reached();
}
hipError_t launch_compress_select(const double*, const double*, const float*, float*, int32_t*, long long, int, int,
                                  int, hipStream_t, const uint16_t*, const float*) {
  return reached();
}
hipError_t launch_fine(const uint16_t*, const uint16_t*, const uint16_t*, const float*, const float*, const int32_t*,
                       float*, long long, int, int, int, int, int, hipStream_t, const float*, float*, float*,
                       uint16_t*, int, const float*) {
  return reached();
}
bool fine_tiled(int, int, int) { return true; }
hipError_t launch_sel_bound(const int32_t*, const float*, float*, long long, int, int, hipStream_t) {
  return reached();
}
hipError_t launch_layer_in(const uint16_t*, const uint16_t*, long long, int, int, int, int, uint16_t*, uint16_t*,
                           uint16_t*, float*, hipStream_t) {
  return reached();
}
hipError_t launch_layer_out(const float*, const uint16_t*, const uint16_t*, long long, int, int, int, int, uint16_t*,
                            hipStream_t) {
  return reached();
}
hipError_t launch_layer_out_merged(const uint16_t*, const uint16_t*, const uint16_t*, long long, int, int, int, int,
                                   uint16_t*, hipStream_t) {
  return reached();
}
hipError_t launch_coarsen(const uint16_t*, float*, long long, int, int, int, hipStream_t) { return reached(); }
hipError_t launch_interp(const uint16_t*, const uint16_t*, const float*, const int32_t*, const float*, long long, int,
                         int, int, int, float*, float4*, hipStream_t) {
  return reached();
}
hipError_t launch_backward(const BwdLaunch&, hipStream_t) { return reached(); }
hipError_t scratch_buffer(void**) { return reached(); }

}  // namespace mosaic
