"""CPU oracle for the NVFP4 W4A4 path — TEST INFRASTRUCTURE ONLY.

This package is the slow, plain, obviously-correct reference that the HIP
library is checked against.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` may import it.  The product path
(``nvfp4_w4a4_block_02_amd``) never imports, calls or links anything here, and
nothing here imports the product path: the two share no code.

Arithmetic contract (what every function below follows):

* element-wise scale/encode math is IEEE float32 NumPy (round-to-nearest-even,
  no FMA contraction, subnormals kept);
* decoded operands are exact and GEMMs are summed in float64;
* bf16 inputs arrive as uint16 bit patterns and are widened exactly.

Sources.  The format is defined by the LongLive-2.0 pages:

* neurohive.io, "LongLive-2.0: NVIDIA научила модель генерировать длинное видео
  в реальном времени с квантованием NVFP4", section "Ключевые компоненты
  LongLive-2.0" / NVFP4 paragraph: E2M1 elements (2 exponent bits, 1 mantissa
  bit) with a block scale per 16 elements and a per-tensor scale; weights and
  activations of the DiT linear layers are quantized; weight gradients pass
  through a random Hadamard transform (RHT) first.
* tailorednewshub.com, "LongLive-2.0: Infraestructura paralela NVFP4 para video
  largo", section "Entrenamiento NVFP4": the block scale is FP8 and the tensor
  scale FP32; RHT is applied before quantization on gradient-sensitive paths.
  Section "Inferencia W4A4 NVFP4": FP4 GEMMs replace the BF16 GEMMs and the KV
  cache uses the same format (about 3.6x smaller than bf16), with an adaptive
  scale selection named Four Over Six (``four_over_six.py`` states the
  reading).
* hyper.ai summary of the LongLive-2.0 paper, section "方法": the KV cache is
  quantized per block of eight frames and rebuilt by a parallel dequant kernel.
* 171host.com, "LongLive 2.0 技术拆解", section 2.2: attention runs over 9
  local latent frames plus 3 sink frames kept in the cache, frame-causally
  (``attention.py`` states the reading).

Everything finer (E4M3 as the FP8 flavour, the scale recipe, rounding, nibble
order, layouts, the RHT normalisation) is a reading where the pages are silent;
each function states the reading it implements.

Parity status: every function here is pinned by ``tests/test_oracle_*.py``
against closed forms, hand-worked blocks (``tests/golden/``), exact rational
arithmetic or library routines; none is "parity unpinned".
"""

from .formats import (  # noqa: F401
    E2M1_MAGNITUDES,
    E4M3_MAX,
    E2M1_MAX,
    GLOBAL_MAX,
    e2m1_value,
    e4m3_value,
    f32_to_e4m3,
    f32_to_e2m1,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
)
from .codec import (  # noqa: F401
    QTensor,
    amax,
    tensor_scale,
    block_scales,
    encode,
    quantize,
    quantize_with_amax,
    dequantize,
    decode_exact,
    kv_quantize,
    kv_dequantize,
)
from .rht import hadamard16, sign_vector, rht16_rows, rht16_quantize  # noqa: F401
from .gemm import gemm_ref, gelu_tanh  # noqa: F401
from .train import linear_train_ref  # noqa: F401
from .attention import decode_kv, key_visibility, window_attention_ref  # noqa: F401
from .four_over_six import (  # noqa: F401
    block_scales_to,
    block_sq_error,
    quantize_4over6,
    quantize_4over6_with_amax,
    kv_quantize_4over6,
)
