// Stand-ins for the device launchers, for the host-only sanitizer build of
// the C ABI (qmv_api.cpp). No GPU code is linked: every launcher records
// that it was reached and returns kStubLaunch, which the API reports as
// QMV_ERR_HIP. A call that passes validation therefore ends in QMV_ERR_HIP
// with the stub's message; a call that fails validation never gets here.
#include "qmv_common.h"

namespace qmv {

int g_stub_launches = 0;
constexpr int kStubLaunch = 9999;

static int reached() {
    ++g_stub_launches;
    return kStubLaunch;
}

int launch_qmv_norm(const LaunchParams&, const NormArgs&, void*) { return reached(); }
int launch_moe_gate_up(const LaunchParams&, const MoeArgs&, void*) { return reached(); }
int launch_zero_fill(void*, int64_t, void*) { return reached(); }
int launch_moe_down(const LaunchParams&, const MoeArgs&, void*) { return reached(); }
int launch_qvm(const QvmParams&, void*) { return reached(); }
int launch_qmm(const QmmParams&, void*) { return reached(); }
int launch_quantize(const QuantParams&, void*) { return reached(); }
int launch_qmv(const LaunchParams&, void*) { return reached(); }
int launch_gather(const LaunchParams&, void*) { return reached(); }
int launch_unpack_device(const uint8_t*, int64_t, int64_t, int, uint8_t*, void*) {
    return reached();
}
int launch_dequant_device(const LaunchParams&, float*, void*) { return reached(); }
const char* hip_error_string(int err) { return err == kStubLaunch ? "stub launch" : "?"; }
int scratch_for_current_device(void** out) {
    static unsigned char host_stand_in[256];
    *out = host_stand_in;
    return 0;
}

}  // namespace qmv
