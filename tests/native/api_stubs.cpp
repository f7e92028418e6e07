// Stand-ins for the library's device launchers, for building the C ABI's host code alone
// (argument checks, launch-argument filling) under sanitizers: each records the call and
// returns success without touching any buffer.
#include "tq_internal.h"

namespace tq {

int g_launches = 0;
AppendArgs g_append;
DecodeArgs g_decode;
MergeArgs g_merge;

hipError_t launch_append(const AppendArgs& a, int, int, bool, bool, int, int, hipStream_t) {
  g_append = a;
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_append_kv(const AppendArgs& ak, const AppendArgs&, int, int, int, bool, int, int, hipStream_t) {
  g_append = ak;
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_decode(const DecodeArgs& a, int, int, int, bool, bool, hipStream_t) {
  g_decode = a;
  ++g_launches;
  return hipSuccess;
}
hipError_t launch_dense(const DenseArgs&, bool, bool, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_dense_mfma(const DenseArgs&, bool, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_zip_compress(const ZipCompressArgs&, int, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_zip_attention(const ZipAttnArgs&, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_gtq_quantize(const GtqQuantArgs&, bool, int, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_gtq_attention(const GtqAttnArgs&, bool, hipStream_t) { ++g_launches; return hipSuccess; }
hipError_t launch_merge(const MergeArgs& a, hipStream_t) {
  g_merge = a;
  ++g_launches;
  return hipSuccess;
}
static float g_static[16];
hipError_t static_partials(float** p) {
  *p = g_static;  // never dereferenced by the host code
  return hipSuccess;
}

}  // namespace tq
