"""Run by tests/test_device_error.py in a child process whose environment
hides every GPU: each entry point of libq8gemm.so gets arguments that pass
all of its host-side checks (aligned stand-in addresses that are never
dereferenced), so each call reaches the one-time device check and must
return Q8_ERR_DEVICE without launching anything.  Prints one line per call;
exits non-zero on the first unexpected status."""
import ctypes
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import int8_block_scaled_amd as q8  # noqa: E402

DEVICE = 6
# Refuse to run if the runtime still sees a device: the calls below would
# then pass every check and launch on stand-in addresses.
hip = ctypes.CDLL("libamdhip64.so")
count = ctypes.c_int(0)
if hip.hipGetDeviceCount(ctypes.byref(count)) == 0 and count.value > 0:
    sys.exit("a GPU is visible (%d devices) despite the hiding environment; not calling"
             % count.value)
L = q8.lib()
P = ctypes.c_void_p(0x100000)          # 16-byte aligned stand-in, never dereferenced
size = ctypes.c_size_t(1 << 40)
calls = {
    "q8_pack_weights": lambda: L.q8_pack_weights(P, 64, 512, P, ctypes.byref(size), None),
    "q8_quantize_act": lambda: L.q8_quantize_act(P, 1, 4, 512, 512, P, P, None),
    "q8_gemm (decode)": lambda: L.q8_gemm(4, 256, 512, P, P, P, P, 256, None),
    "q8_gemm (matrix cores)": lambda: L.q8_gemm(300, 256, 512, P, P, P, P, 256, None),
    "q8_gemm_act": lambda: L.q8_gemm_act(P, 1, 300, 256, 512, 512, P, P, 256, P, P, None),
    "q8_pack_weights_gateup": lambda: L.q8_pack_weights_gateup(P, P, 64, 512, P,
                                                               ctypes.byref(size), None),
    "q8_gemm_swiglu": lambda: L.q8_gemm_swiglu(300, 64, 512, P, P, P, P, P, None),
    "q8_kv3_encode": lambda: L.q8_kv3_encode(P, 1, 16, 128, 128, P, P, None),
    "q8_kv3_decode": lambda: L.q8_kv3_decode(P, P, 16, 128, 1, P, 128, None),
    "q8_attn_pool": lambda: L.q8_attn_pool(P, 100, 512, 4, 128, P, None),
    "q8_attn_select": lambda: L.q8_attn_select(P, P, 4, 2, 2, 128, 2, 2, P, P, None),
    "q8_attn_fwd": lambda: L.q8_attn_fwd(P, P, P, 100, 512, 256, 256, 4, 2, 128, P, P, 4, 1, P,
                                         512, None),
}
for name, call in calls.items():
    st = call()
    print("%s -> %d" % (name, st), flush=True)
    if st != DEVICE:
        sys.exit("%s returned %d, expected Q8_ERR_DEVICE (%d)" % (name, st, DEVICE))
print("all entry points: Q8_ERR_DEVICE")
