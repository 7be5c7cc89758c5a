"""MI355X-native MoE decode/verify round: a HIP library behind a C ABI, with a thin binding.

    from verify_router_gemv_amd import MoeRound
"""
from .binding import (  # noqa: F401
    LIB_PATH,
    MoeRound,
    MoeRoundError,
    load,
    make_config,
    validate_config,
)
